"""Python front end of libsvdq: the same entry points as include/svdq.h.

Host prep functions take and return numpy arrays. Device functions take
torch tensors on a ROCm device and enqueue work on torch's current stream
(or the stream passed in); PyTorch only provides the memory and the stream.
All checks and all arithmetic are done by the library.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import _lib
from ._lib import F16, F32, GROUP, MX_BLOCK, check, lib

# --------------------------------------------------------------------------
# host prep (numpy)


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def channel_absmax(X: np.ndarray) -> np.ndarray:
    X = np.ascontiguousarray(X)
    dt = F16 if X.dtype == np.float16 else F32
    if dt == F32:
        X = _c(X, np.float32)
    M, K = X.shape
    out = np.empty(K, dtype=np.float32)
    check(lib.svdq_channel_absmax(_np_ptr(X), dt, M, K, K, _np_ptr(out)), "svdq_channel_absmax")
    return out


def smoothing_factors(x_absmax: np.ndarray, W: np.ndarray) -> np.ndarray:
    xa = _c(x_absmax, np.float32)
    W = _c(W, np.float32)
    K, N = W.shape
    lam = np.empty(K, dtype=np.float32)
    check(lib.svdq_smoothing_factors(_np_ptr(xa), _np_ptr(W), K, N, _np_ptr(lam)),
          "svdq_smoothing_factors")
    return lam


@dataclasses.dataclass
class Prepared:
    """Offline products for one layer, host side. L1t is R x K, L2t is N x R (fp16 bits).
    ``fmt`` "int4": w_scales are the fp16 group scales (N x K/64, as uint16 bits);
    ``fmt`` "mxfp4": w_scales are the E8M0 block exponents (N x K/32, uint8);
    ``fmt`` "w4a16": the weight-only baseline, Q of W itself (rank 0, no smoothing)."""
    K: int
    N: int
    rank: int
    inv_smooth: np.ndarray
    L1t: np.ndarray
    L2t: np.ndarray
    w_codes: np.ndarray
    w_scales: np.ndarray
    sigma: Optional[np.ndarray] = None
    fmt: str = "int4"

    @property
    def L1(self) -> np.ndarray:
        """K x R fp16 view of the factor (a copy)."""
        return np.ascontiguousarray(self.L1t.view(np.float16).T)

    @property
    def L2(self) -> np.ndarray:
        """R x N fp16 (a copy)."""
        return np.ascontiguousarray(self.L2t.view(np.float16).T)

    @property
    def L1p(self) -> Optional[np.ndarray]:
        """L1 packed in the order the device pre-kernel reads it (None at rank 0)."""
        return pack_lowrank_down(self.L1t) if self.rank else None


def pack_lowrank_down(L1t: np.ndarray) -> np.ndarray:
    """svdq_pack_lowrank_down: R x K fp16 bits -> R*K fp16 bits in operand order."""
    L1t = _c(L1t, np.uint16)
    R, K = L1t.shape
    out = np.empty(R * K, dtype=np.uint16)
    check(lib.svdq_pack_lowrank_down(_np_ptr(L1t), K, R, _np_ptr(out)), "svdq_pack_lowrank_down")
    return out


def pack_lowrank(L1: np.ndarray, L2: np.ndarray):
    """svdq_pack_lowrank: the canonical factors L1 (K x R) and L2 (R x N), fp16 bits
    -> (L1p, R*K fp16 bits in K1's operand order; L2t, N x R fp16 bits)."""
    L1 = _c(L1, np.uint16)
    L2 = _c(L2, np.uint16)
    K, R = L1.shape
    R2, N = L2.shape
    if R2 != R:
        raise ValueError(f"L1 is {K} x {R} but L2 is {R2} x {N}")
    L1p = np.empty(R * K, dtype=np.uint16)
    L2t = np.empty((N, R), dtype=np.uint16)
    check(lib.svdq_pack_lowrank(_np_ptr(L1), _np_ptr(L2), K, N, R, _np_ptr(L1p), _np_ptr(L2t)),
          "svdq_pack_lowrank")
    return L1p, L2t


def prepare_weights(W: np.ndarray, lam: np.ndarray, rank: int, want_sigma: bool = False) -> Prepared:
    W = _c(W, np.float32)
    lam = _c(lam, np.float32)
    K, N = W.shape
    inv = np.empty(K, dtype=np.float32)
    L1t = np.empty((rank, K), dtype=np.uint16)
    L2t = np.empty((N, rank), dtype=np.uint16)
    wc = np.empty((N, K // 2), dtype=np.uint8)
    ws = np.empty((N, K // GROUP), dtype=np.uint16)
    sig = np.empty(min(K, N), dtype=np.float64) if want_sigma else None
    check(lib.svdq_prepare_weights(_np_ptr(W), _np_ptr(lam), K, N, rank, GROUP, _np_ptr(inv),
                                   _np_ptr(L1t) if rank else None, _np_ptr(L2t) if rank else None,
                                   _np_ptr(wc), _np_ptr(ws), _np_ptr(sig)),
          "svdq_prepare_weights")
    return Prepared(K, N, rank, inv, L1t, L2t, wc, ws, sig)


def prepare_weights_mx(W: np.ndarray, lam: np.ndarray, rank: int,
                       want_sigma: bool = False) -> Prepared:
    """svdq_prepare_weights_mx: the same split, residual in MXFP4 (fmt "mxfp4")."""
    W = _c(W, np.float32)
    lam = _c(lam, np.float32)
    K, N = W.shape
    inv = np.empty(K, dtype=np.float32)
    L1t = np.empty((rank, K), dtype=np.uint16)
    L2t = np.empty((N, rank), dtype=np.uint16)
    wc = np.empty((N, K // 2), dtype=np.uint8)
    we = np.empty((N, K // MX_BLOCK), dtype=np.uint8)
    sig = np.empty(min(K, N), dtype=np.float64) if want_sigma else None
    check(lib.svdq_prepare_weights_mx(_np_ptr(W), _np_ptr(lam), K, N, rank, _np_ptr(inv),
                                      _np_ptr(L1t) if rank else None,
                                      _np_ptr(L2t) if rank else None, _np_ptr(wc), _np_ptr(we),
                                      _np_ptr(sig)),
          "svdq_prepare_weights_mx")
    return Prepared(K, N, rank, inv, L1t, L2t, wc, we, sig, fmt="mxfp4")


def mx_codes_tiled_bytes(rows: int, K: int) -> int:
    return int(lib.svdq_mx_codes_tiled_bytes(rows, K))


def mx_exps_tiled_bytes(rows: int, K: int) -> int:
    return int(lib.svdq_mx_exps_tiled_bytes(rows, K))


def pack_mx_tiles(codes: np.ndarray, e8m0: np.ndarray, K: int):
    """svdq_pack_mx_tiles: canonical MXFP4 codes (rows x K/2) and exponents
    (rows x K/32) -> the tiled device layouts (flat uint8 arrays)."""
    codes = _c(codes, np.uint8)
    e8m0 = _c(e8m0, np.uint8)
    rows = codes.shape[0]
    ct = np.empty(mx_codes_tiled_bytes(rows, K), dtype=np.uint8)
    et = np.empty(mx_exps_tiled_bytes(rows, K), dtype=np.uint8)
    check(lib.svdq_pack_mx_tiles(_np_ptr(codes), _np_ptr(e8m0), rows, K, _np_ptr(ct), _np_ptr(et)),
          "svdq_pack_mx_tiles")
    return ct, et


def prepare_weights_w4a16(W: np.ndarray) -> Prepared:
    """svdq_prepare_weights_w4a16: the 4-bit weight-only baseline's weights
    (the group quantizer on W itself; fmt "w4a16", rank 0)."""
    W = _c(W, np.float32)
    K, N = W.shape
    wc = np.empty((N, K // 2), dtype=np.uint8)
    ws = np.empty((N, K // GROUP), dtype=np.uint16)
    check(lib.svdq_prepare_weights_w4a16(_np_ptr(W), K, N, _np_ptr(wc), _np_ptr(ws)),
          "svdq_prepare_weights_w4a16")
    return Prepared(K, N, 0, np.ones(K, dtype=np.float32), np.empty((0, K), np.uint16),
                    np.empty((N, 0), np.uint16), wc, ws, None, fmt="w4a16")


def pack_w4a16_tiles(w_codes: np.ndarray, w_scales: np.ndarray, K: int):
    """svdq_pack_w4a16_tiles: canonical weight-only codes and fp16 scale bits ->
    the tiled device layouts (flat uint8 codes, flat uint16 scale bits)."""
    w_codes = _c(w_codes, np.uint8)
    w_scales = _c(w_scales, np.uint16)
    N = w_codes.shape[0]
    ct = np.empty(int(lib.svdq_w4a16_codes_tiled_bytes(N, K)), dtype=np.uint8)
    st = np.empty(int(lib.svdq_w4a16_scales_tiled_bytes(N, K)) // 2, dtype=np.uint16)
    check(lib.svdq_pack_w4a16_tiles(_np_ptr(w_codes), _np_ptr(w_scales), N, K, _np_ptr(ct),
                                    _np_ptr(st)), "svdq_pack_w4a16_tiles")
    return ct, st


def concat_lora(prep: Prepared, lam: np.ndarray, A: np.ndarray, B: np.ndarray,
                scale: float = 1.0) -> Prepared:
    A = _c(A, np.float16).view(np.uint16)
    B = _c(B, np.float16).view(np.uint16)
    lam = _c(lam, np.float32)
    K, N, r = prep.K, prep.N, prep.rank
    rl = A.shape[1]
    L1o = np.empty((r + rl, K), dtype=np.uint16)
    L2o = np.empty((N, r + rl), dtype=np.uint16)
    check(lib.svdq_concat_lora(_np_ptr(prep.L1t) if r else None, _np_ptr(prep.L2t) if r else None,
                               K, N, r, _np_ptr(lam), _np_ptr(A), _np_ptr(B), rl, float(scale),
                               _np_ptr(L1o), _np_ptr(L2o)), "svdq_concat_lora")
    return dataclasses.replace(prep, rank=r + rl, L1t=L1o, L2t=L2o)


# --------------------------------------------------------------------------
# device entry points (torch tensors)
#
# The kernels trust the shapes they are given: a weight buffer shorter than
# K and N imply, or an output narrower than the layer, would be read or
# written past its end. So every entry point checks, before the library call,
# that each tensor's shape, dtype, size and strides agree with the others,
# then that all of them sit on one GPU (that check comes last, so the others
# can be exercised without a GPU). Violations raise ValueError or TypeError.


def _torch():
    import torch
    return torch


def _tp(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


_BYTES = ("uint8", "int8")
_HALF = ("float16", "int16", "uint16")        # fp16 values or their bit patterns
_F32 = ("float32",)
_XY = ("float16", "float32")


def _dtname(t) -> str:
    return str(t.dtype).replace("torch.", "")


def _buf(name, t, dtypes, nbytes=None, min_bytes=None, contiguous=True):
    """A flat buffer: dtype in `dtypes`, exactly `nbytes` or at least `min_bytes`."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if _dtname(t) not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    size = t.numel() * t.element_size()
    if nbytes is not None and size != nbytes:
        raise ValueError(f"{name}: {size} bytes, expected {nbytes}")
    if min_bytes is not None and size < min_bytes:
        raise ValueError(f"{name}: {size} bytes, at least {min_bytes} needed")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _mat(name, t, rows, cols, dtypes=_XY):
    """A row-major matrix of `rows` x `cols` with unit inner stride (any row stride >= cols)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if _dtname(t) not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != 2 or (rows is not None and t.shape[0] != rows) or (
            cols is not None and t.shape[1] != cols):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected ({rows}, {cols})")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: the inner stride must be 1, got {t.stride(1)}")
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError(f"{name}: row stride {t.stride(0)} < {t.shape[1]} columns")
    return t


def _on_gpu(*ts):
    devs = {(t.device.type, t.device.index) for t in ts if t is not None}
    if any(d[0] != "cuda" for d in devs):
        raise ValueError("every tensor must be on a GPU (device memory)")
    if len(devs) > 1:
        raise ValueError(f"tensors on several devices: {sorted(devs)}")


def _groups(K: int) -> int:
    if K < GROUP or K % GROUP:
        raise ValueError(f"K={K}: need a positive multiple of {GROUP}")
    return K // GROUP


def _bias(bias, N):
    if bias is not None:
        _buf("bias", bias, _F32, nbytes=4 * N)


def _act_side(M, K, R, a_codes, a_scales, D, mx=False):
    """Checks of the activation-side buffers written by K1 and read by K2."""
    G = _groups(K)
    if mx:
        _buf("a_codes_t", a_codes, _BYTES, min_bytes=mx_codes_tiled_bytes(M, K))
        _buf("a_exps_t", a_scales, _BYTES, min_bytes=mx_exps_tiled_bytes(M, K))
    else:
        _buf("a_codes", a_codes, _BYTES, min_bytes=M * K // 2)
        _buf("a_scales", a_scales, _HALF, min_bytes=2 * M * G)
    if R:
        if mx:
            _buf("D_t", D, _HALF, min_bytes=int4_d_tiled_bytes(M, R))
        else:
            _buf("D", D, _F32, min_bytes=4 * M * R)


def _weights(N, K, R, w_codes, w_scales, L2t, mx=False):
    G = _groups(K)
    if mx:
        _buf("w_codes_t", w_codes, _BYTES, nbytes=mx_codes_tiled_bytes(N, K))
        _buf("w_exps_t", w_scales, _BYTES, nbytes=mx_exps_tiled_bytes(N, K))
    else:
        _buf("w_codes", w_codes, _BYTES, nbytes=N * K // 2)
        _buf("w_scales", w_scales, _HALF, nbytes=2 * N * G)
    if R:
        _buf("L2t", L2t, _HALF, nbytes=2 * N * R)


def _down(K, R, inv_smooth, L1p):
    _buf("inv_smooth", inv_smooth, _F32, nbytes=4 * K)
    if R:
        _buf("L1p", L1p, _HALF, nbytes=2 * R * K)


def quantize_act_lowrank_down(X, inv_smooth, L1p, R: int, a_codes, a_scales, D, stream=None):
    _mat("X", X, None, None)
    M, K = X.shape
    _down(K, R, inv_smooth, L1p)
    _act_side(M, K, R, a_codes, a_scales, D)
    _on_gpu(X, inv_smooth, L1p if R else None, a_codes, a_scales, D if R else None)
    check(lib.svdq_quantize_act_lowrank_down(_tp(X), _dt(X), M, K, X.stride(0), _tp(inv_smooth),
                                             _tp(L1p) if R else None, R, GROUP, _tp(a_codes),
                                             _tp(a_scales), _tp(D) if R else None, _stream(stream)),
          "svdq_quantize_act_lowrank_down")


def _act(activation) -> int:
    if activation is None or activation == "none":
        return _lib.ACT_NONE
    if activation == "gelu_tanh":
        return _lib.ACT_GELU_TANH
    raise ValueError(f"unknown activation {activation!r}")


def w4a4_gemm_lowrank_up(a_codes, a_scales, w_codes, w_scales, D, L2t, R: int, bias, Y, K: int,
                         stream=None, activation=None):
    _mat("Y", Y, None, None)
    M, N = Y.shape
    _act_side(M, K, R, a_codes, a_scales, D)
    _weights(N, K, R, w_codes, w_scales, L2t)
    _bias(bias, N)
    _on_gpu(a_codes, a_scales, w_codes, w_scales, D if R else None, L2t if R else None, bias, Y)
    check(lib.svdq_w4a4_gemm_lowrank_up(_tp(a_codes), _tp(a_scales), _tp(w_codes), _tp(w_scales),
                                        _tp(D) if R else None, _tp(L2t) if R else None, R, _tp(bias),
                                        _tp(Y), _dt(Y), M, N, K, Y.stride(0), GROUP,
                                        _act(activation), _stream(stream)),
          "svdq_w4a4_gemm_lowrank_up")


def linear_workspace_bytes(M: int, K: int, R: int) -> int:
    return int(lib.svdq_linear_workspace_bytes(M, K, R, GROUP))


def _layer_io(X, Y, K=None, N=None):
    _mat("X", X, None, K)
    M = X.shape[0]
    _mat("Y", Y, M, N)
    return M, X.shape[1], Y.shape[1]


def linear(X, inv_smooth, L1p, L2t, R: int, w_codes, w_scales, bias, Y, ws, stream=None,
           activation=None):
    M, K, N = _layer_io(X, Y)
    _down(K, R, inv_smooth, L1p)
    _weights(N, K, R, w_codes, w_scales, L2t)
    _bias(bias, N)
    _buf("ws", ws, _BYTES + _HALF + _F32, min_bytes=linear_workspace_bytes(M, K, R))
    _on_gpu(X, inv_smooth, L1p if R else None, L2t if R else None, w_codes, w_scales, bias, Y, ws)
    check(lib.svdq_linear(_tp(X), _dt(X), X.stride(0), _tp(inv_smooth), _tp(L1p) if R else None,
                          _tp(L2t) if R else None, R, _tp(w_codes), _tp(w_scales), _tp(bias), _tp(Y),
                          _dt(Y), Y.stride(0), M, K, N, GROUP, _tp(ws), ws.numel() * ws.element_size(),
                          _act(activation), _stream(stream)), "svdq_linear")


def linear_canonical_workspace_bytes(M: int, K: int, N: int, R: int) -> int:
    return int(lib.svdq_linear_canonical_workspace_bytes(M, K, N, R, GROUP))


def linear_canonical(X, inv_smooth, L1, L2, R: int, w_codes, w_scales, bias, Y, ws, stream=None,
                     activation=None):
    """svdq_linear_canonical: the layer with the low-rank factors as L1 (K x R) and
    L2 (R x N) fp16 device arrays."""
    M, K, N = _layer_io(X, Y)
    _buf("inv_smooth", inv_smooth, _F32, nbytes=4 * K)
    if R:
        _buf("L1", L1, _HALF, nbytes=2 * K * R)
        _buf("L2", L2, _HALF, nbytes=2 * R * N)
    _weights(N, K, 0, w_codes, w_scales, None)
    _bias(bias, N)
    _buf("ws", ws, _BYTES + _HALF + _F32, min_bytes=linear_canonical_workspace_bytes(M, K, N, R))
    _on_gpu(X, inv_smooth, L1 if R else None, L2 if R else None, w_codes, w_scales, bias, Y, ws)
    check(lib.svdq_linear_canonical(_tp(X), _dt(X), X.stride(0), _tp(inv_smooth),
                                    _tp(L1) if R else None, _tp(L2) if R else None, R,
                                    _tp(w_codes), _tp(w_scales), _tp(bias), _tp(Y), _dt(Y),
                                    Y.stride(0), M, K, N, GROUP, _tp(ws),
                                    ws.numel() * ws.element_size(), _act(activation),
                                    _stream(stream)), "svdq_linear_canonical")


def int4_act_tiled_bytes(M: int, K: int) -> int:
    return int(lib.svdq_int4_act_tiled_bytes(M, K))


def int4_act_scales_tiled_bytes(M: int, K: int) -> int:
    return int(lib.svdq_int4_act_scales_tiled_bytes(M, K))


def int4_d_tiled_bytes(M: int, R: int) -> int:
    return int(lib.svdq_int4_d_tiled_bytes(M, R))


def int4_w_codes_tiled_bytes(N: int, K: int) -> int:
    return int(lib.svdq_int4_w_codes_tiled_bytes(N, K))


def int4_w_scales_tiled_bytes(N: int, K: int) -> int:
    return int(lib.svdq_int4_w_scales_tiled_bytes(N, K))


def pack_w4a4_tiles(w_codes: np.ndarray, w_scales: np.ndarray, K: int):
    """svdq_pack_w4a4_tiles: canonical INT4 weight codes and fp16 scale bits -> the
    tiled layouts of the tiled path (flat uint8 codes, flat fp32 scale pairs)."""
    w_codes = _c(w_codes, np.uint8)
    w_scales = _c(w_scales, np.uint16)
    N = w_codes.shape[0]
    ct = np.empty(int4_w_codes_tiled_bytes(N, K), dtype=np.uint8)
    st = np.empty(int4_w_scales_tiled_bytes(N, K) // 4, dtype=np.float32)
    check(lib.svdq_pack_w4a4_tiles(_np_ptr(w_codes), _np_ptr(w_scales), N, K, _np_ptr(ct),
                                   _np_ptr(st)), "svdq_pack_w4a4_tiles")
    return ct, st


def _act_side_tiled(M, K, R, a_ops_t, a_scales_t, D_t):
    _groups(K)
    _buf("a_ops_t", a_ops_t, _BYTES, min_bytes=int4_act_tiled_bytes(M, K))
    _buf("a_scales_t", a_scales_t, _F32, min_bytes=int4_act_scales_tiled_bytes(M, K))
    if R:
        _buf("D_t", D_t, _HALF, min_bytes=int4_d_tiled_bytes(M, R))


def _weights_tiled(N, K, R, w_codes_t, w_scales_t, L2t):
    _groups(K)
    _buf("w_codes_t", w_codes_t, _BYTES, nbytes=int4_w_codes_tiled_bytes(N, K))
    _buf("w_scales_t", w_scales_t, _F32, nbytes=int4_w_scales_tiled_bytes(N, K))
    if R:
        _buf("L2t", L2t, _HALF, nbytes=2 * N * R)


def quantize_act_workspace_bytes(M: int, K: int, R: int) -> int:
    """Bytes of the optional pre-kernel workspace (tiled INT4 and MXFP4) on the
    current device; 0 when the shape does not split."""
    return int(lib.svdq_quantize_act_workspace_bytes(M, K, R))


def _opt_ws(workspace):
    """(pointer, bytes) of an optional workspace (the pre-kernels', the tiled GEMM's)."""
    if workspace is None:
        return None, 0
    if workspace.dtype != _torch().uint8 or not workspace.is_contiguous():
        raise ValueError("workspace: a contiguous uint8 tensor")
    return _tp(workspace), workspace.numel()


def quantize_act_lowrank_down_tiled(X, inv_smooth, L1p, R: int, a_ops_t, a_scales_t, D_t,
                                    stream=None, workspace=None):
    """K1 writing the tiled activation operands, fp32 scales and fp16 D_t.
    workspace: None, or quantize_act_workspace_bytes(M, K, R) bytes (uint8) on
    the same device, with which long rows run split."""
    D = D_t
    _mat("X", X, None, None)
    M, K = X.shape
    _down(K, R, inv_smooth, L1p)
    _act_side_tiled(M, K, R, a_ops_t, a_scales_t, D)
    _on_gpu(X, inv_smooth, L1p if R else None, a_ops_t, a_scales_t, D if R else None, workspace)
    wp, wb = _opt_ws(workspace)
    check(lib.svdq_quantize_act_lowrank_down_tiled(_tp(X), _dt(X), M, K, X.stride(0),
                                                   _tp(inv_smooth), _tp(L1p) if R else None, R,
                                                   _tp(a_ops_t), _tp(a_scales_t),
                                                   _tp(D) if R else None, wp, wb,
                                                   _stream(stream)),
          "svdq_quantize_act_lowrank_down_tiled")


def gemm_tiled_workspace_bytes(M: int, N: int, K: int) -> int:
    """Bytes of the tiled GEMM's optional workspace on the current device (its
    split along K); 0 when the shape does not split."""
    return int(lib.svdq_gemm_tiled_workspace_bytes(M, N, K))


def w4a4_gemm_lowrank_up_tiled(a_ops_t, a_scales_t, w_codes_t, w_scales_t, D_t, L2t, R: int, bias,
                               Y, K: int, stream=None, activation=None, workspace=None):
    """K2 on the tiled layouts (D_t: the pre-kernel's fp16 D in operand order).
    workspace: None, or gemm_tiled_workspace_bytes(M, N, K) bytes (uint8) on the
    same device, with which an under-filled long-K GEMM runs split along K."""
    D = D_t
    _mat("Y", Y, None, None)
    M, N = Y.shape
    _act_side_tiled(M, K, R, a_ops_t, a_scales_t, D)
    _weights_tiled(N, K, R, w_codes_t, w_scales_t, L2t)
    _bias(bias, N)
    _on_gpu(a_ops_t, a_scales_t, w_codes_t, w_scales_t, D if R else None, L2t if R else None, bias,
            Y, workspace)
    wp, wb = _opt_ws(workspace)
    check(lib.svdq_w4a4_gemm_lowrank_up_tiled(_tp(a_ops_t), _tp(a_scales_t), _tp(w_codes_t),
                                              _tp(w_scales_t), _tp(D) if R else None,
                                              _tp(L2t) if R else None, R, _tp(bias), _tp(Y),
                                              _dt(Y), M, N, K, Y.stride(0), _act(activation),
                                              wp, wb, _stream(stream)),
          "svdq_w4a4_gemm_lowrank_up_tiled")


def linear_tiled_workspace_bytes(M: int, K: int, R: int) -> int:
    return int(lib.svdq_linear_tiled_workspace_bytes(M, K, R))


def linear_tiled(X, inv_smooth, L1p, L2t, R: int, w_codes_t, w_scales_t, bias, Y, ws, stream=None,
                 activation=None):
    """The whole INT4 layer on the tiled path (weights from pack_w4a4_tiles)."""
    M, K, N = _layer_io(X, Y)
    _down(K, R, inv_smooth, L1p)
    _weights_tiled(N, K, R, w_codes_t, w_scales_t, L2t)
    _bias(bias, N)
    _buf("ws", ws, _BYTES + _HALF + _F32, min_bytes=linear_tiled_workspace_bytes(M, K, R))
    _on_gpu(X, inv_smooth, L1p if R else None, L2t if R else None, w_codes_t, w_scales_t, bias, Y,
            ws)
    check(lib.svdq_linear_tiled(_tp(X), _dt(X), X.stride(0), _tp(inv_smooth),
                                _tp(L1p) if R else None, _tp(L2t) if R else None, R,
                                _tp(w_codes_t), _tp(w_scales_t), _tp(bias), _tp(Y), _dt(Y),
                                Y.stride(0), M, K, N, _tp(ws), ws.numel() * ws.element_size(),
                                _act(activation), _stream(stream)), "svdq_linear_tiled")


def linear_noalloc(X, inv_smooth, L1p, L2t, R: int, w_codes, w_scales, bias, Y, stream=None,
                   activation=None):
    """svdq_linear with the intermediates in the library's static device buffer
    (no workspace, no allocation; calls that overlap on one GPU race)."""
    M, K, N = _layer_io(X, Y)
    _down(K, R, inv_smooth, L1p)
    _weights(N, K, R, w_codes, w_scales, L2t)
    _bias(bias, N)
    _on_gpu(X, inv_smooth, L1p if R else None, L2t if R else None, w_codes, w_scales, bias, Y)
    check(lib.svdq_linear_noalloc(_tp(X), _dt(X), X.stride(0), _tp(inv_smooth),
                                  _tp(L1p) if R else None, _tp(L2t) if R else None, R,
                                  _tp(w_codes), _tp(w_scales), _tp(bias), _tp(Y), _dt(Y),
                                  Y.stride(0), M, K, N, GROUP, _act(activation), _stream(stream)),
          "svdq_linear_noalloc")


def quantize_act_lowrank_down_mx(X, inv_smooth, L1p, R: int, a_codes_t, a_exps_t, D, stream=None,
                                 workspace=None):
    """K1-MX; a_codes_t / a_exps_t: device buffers of mx_codes_tiled_bytes(M, K) and
    mx_exps_tiled_bytes(M, K) bytes (tiled layouts); D: D_t, fp16 in the
    up-projection's operand order (int4_d_tiled_bytes(M, R) bytes); workspace:
    as for quantize_act_lowrank_down_tiled."""
    _mat("X", X, None, None)
    M, K = X.shape
    _down(K, R, inv_smooth, L1p)
    _act_side(M, K, R, a_codes_t, a_exps_t, D, mx=True)
    _on_gpu(X, inv_smooth, L1p if R else None, a_codes_t, a_exps_t, D if R else None, workspace)
    wp, wb = _opt_ws(workspace)
    check(lib.svdq_quantize_act_lowrank_down_mx(_tp(X), _dt(X), M, K, X.stride(0), _tp(inv_smooth),
                                                _tp(L1p) if R else None, R, _tp(a_codes_t),
                                                _tp(a_exps_t), _tp(D) if R else None, wp, wb,
                                                _stream(stream)),
          "svdq_quantize_act_lowrank_down_mx")


def mx_gemm_lowrank_up(a_codes_t, a_exps_t, w_codes_t, w_exps_t, D, L2t, R: int, bias, Y, K: int,
                       stream=None, activation=None):
    """K2-MX on the tiled activation and weight codes and exponents."""
    _mat("Y", Y, None, None)
    M, N = Y.shape
    _act_side(M, K, R, a_codes_t, a_exps_t, D, mx=True)
    _weights(N, K, R, w_codes_t, w_exps_t, L2t, mx=True)
    _bias(bias, N)
    _on_gpu(a_codes_t, a_exps_t, w_codes_t, w_exps_t, D if R else None, L2t if R else None, bias, Y)
    check(lib.svdq_mx_gemm_lowrank_up(_tp(a_codes_t), _tp(a_exps_t), _tp(w_codes_t), _tp(w_exps_t),
                                      _tp(D) if R else None, _tp(L2t) if R else None, R, _tp(bias),
                                      _tp(Y), _dt(Y), M, N, K, Y.stride(0), _act(activation),
                                      _stream(stream)),
          "svdq_mx_gemm_lowrank_up")


def linear_mx_workspace_bytes(M: int, K: int, R: int) -> int:
    return int(lib.svdq_linear_mx_workspace_bytes(M, K, R))


def linear_mx(X, inv_smooth, L1p, L2t, R: int, w_codes_t, w_exps_t, bias, Y, ws, stream=None,
              activation=None):
    """The whole MXFP4 layer; the weights in the tiled layouts (pack_mx_tiles)."""
    M, K, N = _layer_io(X, Y)
    _down(K, R, inv_smooth, L1p)
    _weights(N, K, R, w_codes_t, w_exps_t, L2t, mx=True)
    _bias(bias, N)
    _buf("ws", ws, _BYTES + _HALF + _F32, min_bytes=linear_mx_workspace_bytes(M, K, R))
    _on_gpu(X, inv_smooth, L1p if R else None, L2t if R else None, w_codes_t, w_exps_t, bias, Y,
            ws)
    check(lib.svdq_linear_mx(_tp(X), _dt(X), X.stride(0), _tp(inv_smooth),
                             _tp(L1p) if R else None, _tp(L2t) if R else None, R, _tp(w_codes_t),
                             _tp(w_exps_t), _tp(bias), _tp(Y), _dt(Y), Y.stride(0), M, K, N, _tp(ws),
                             ws.numel() * ws.element_size(), _act(activation), _stream(stream)),
          "svdq_linear_mx")


def w4a16_x_tiled_bytes(M: int, K: int) -> int:
    return int(lib.svdq_w4a16_x_tiled_bytes(M, K))


def _w4a16_weights(N, K, w_codes_t, w_scales_t):
    _groups(K)
    _buf("w_codes_t", w_codes_t, _BYTES, nbytes=int(lib.svdq_w4a16_codes_tiled_bytes(N, K)))
    _buf("w_scales_t", w_scales_t, _HALF, nbytes=int(lib.svdq_w4a16_scales_tiled_bytes(N, K)))


def w4a16_tile_activation(X, x_t, stream=None):
    """X (fp16 or fp32, M x K) -> x_t (w4a16_x_tiled_bytes(M, K) bytes), the tiled fp16 layout."""
    _mat("X", X, None, None)
    M, K = X.shape
    _groups(K)
    _buf("x_t", x_t, _BYTES + _HALF, min_bytes=w4a16_x_tiled_bytes(M, K))
    _on_gpu(X, x_t)
    check(lib.svdq_w4a16_tile_activation(_tp(X), _dt(X), M, K, X.stride(0), _tp(x_t),
                                         _stream(stream)), "svdq_w4a16_tile_activation")


def w4a16_gemm(x_t, w_codes_t, w_scales_t, bias, Y, K: int, stream=None):
    _mat("Y", Y, None, None)
    M, N = Y.shape
    _groups(K)
    _buf("x_t", x_t, _BYTES + _HALF, min_bytes=w4a16_x_tiled_bytes(M, K))
    _w4a16_weights(N, K, w_codes_t, w_scales_t)
    _bias(bias, N)
    _on_gpu(x_t, w_codes_t, w_scales_t, bias, Y)
    check(lib.svdq_w4a16_gemm(_tp(x_t), _tp(w_codes_t), _tp(w_scales_t), _tp(bias), _tp(Y), _dt(Y),
                              M, N, K, Y.stride(0), _stream(stream)), "svdq_w4a16_gemm")


def linear_w4a16(X, w_codes_t, w_scales_t, bias, Y, ws, stream=None):
    """The weight-only baseline layer (tiling of X into ws, then the GEMM)."""
    M, K, N = _layer_io(X, Y)
    _groups(K)
    _w4a16_weights(N, K, w_codes_t, w_scales_t)
    _bias(bias, N)
    _buf("ws", ws, _BYTES + _HALF + _F32, min_bytes=w4a16_x_tiled_bytes(M, K))
    _on_gpu(X, w_codes_t, w_scales_t, bias, Y, ws)
    check(lib.svdq_linear_w4a16(_tp(X), _dt(X), X.stride(0), _tp(w_codes_t), _tp(w_scales_t),
                                _tp(bias), _tp(Y), _dt(Y), Y.stride(0), M, K, N, _tp(ws),
                                ws.numel() * ws.element_size(), _stream(stream)),
          "svdq_linear_w4a16")


# --------------------------------------------------------------------------
# convolutions: the linear layer on the implicit patch matrix of an NHWC image


def conv_out_size(n: int, k: int, stride: int, pad: int) -> int:
    """Output extent of a convolution along one axis."""
    return (n + 2 * pad - k) // stride + 1


def conv_patch_absmax(X: np.ndarray, KH: int, KW: int, stride: int, pad: int) -> np.ndarray:
    """Column maxima of |patch matrix| (length KH*KW*C) for an NHWC image X."""
    X = np.ascontiguousarray(X)
    dt = F16 if X.dtype == np.float16 else F32
    if dt == F32:
        X = _c(X, np.float32)
    B, H, W, Cc = X.shape
    out = np.empty(KH * KW * Cc, dtype=np.float32)
    check(lib.svdq_conv_patch_absmax(_np_ptr(X), dt, B, H, W, Cc, KH, KW, stride, pad,
                                     _np_ptr(out)), "svdq_conv_patch_absmax")
    return out


def _image(X):
    torch = _torch()
    if not isinstance(X, torch.Tensor):
        raise TypeError(f"X: expected a torch tensor, got {type(X).__name__}")
    if _dtname(X) not in _XY:
        raise ValueError(f"X: dtype {X.dtype}, expected one of {_XY}")
    if X.dim() != 4 or not X.is_contiguous():
        raise ValueError(f"X: expected a contiguous NHWC image, got shape {tuple(X.shape)}")
    return X.shape


def _conv_shape(X, KH, KW, stride, pad):
    B, H, W, Cc = _image(X)
    if min(KH, KW, stride) < 1 or pad < 0:
        raise ValueError(f"kernel {KH}x{KW}, stride {stride}, pad {pad}")
    OH, OW = conv_out_size(H, KH, stride, pad), conv_out_size(W, KW, stride, pad)
    if OH < 1 or OW < 1:
        raise ValueError(f"empty output: {OH} x {OW}")
    return B, H, W, Cc, OH, OW, B * OH * OW, KH * KW * Cc


def _conv_out(Y, B, OH, OW, N=None):
    torch = _torch()
    if not isinstance(Y, torch.Tensor):
        raise TypeError(f"Y: expected a torch tensor, got {type(Y).__name__}")
    if _dtname(Y) not in _XY:
        raise ValueError(f"Y: dtype {Y.dtype}, expected one of {_XY}")
    if Y.dim() != 4 or tuple(Y.shape[:3]) != (B, OH, OW) or (N is not None and Y.shape[3] != N) \
            or not Y.is_contiguous():
        raise ValueError(f"Y: expected a contiguous ({B}, {OH}, {OW}, N) output, got "
                         f"{tuple(Y.shape)}")
    return Y.shape[3]


def quantize_act_lowrank_down_conv(X, KH: int, KW: int, stride: int, pad: int, inv_smooth, L1p,
                                   R: int, a_codes, a_scales, D, stream=None):
    """K1 on the patch matrix of the NHWC image X (batch x H x W x C, contiguous)."""
    B, H, W, Cc, OH, OW, M, K = _conv_shape(X, KH, KW, stride, pad)
    _down(K, R, inv_smooth, L1p)
    _act_side(M, K, R, a_codes, a_scales, D)
    _on_gpu(X, inv_smooth, L1p if R else None, a_codes, a_scales, D if R else None)
    check(lib.svdq_quantize_act_lowrank_down_conv(
        _tp(X), _dt(X), B, H, W, Cc, KH, KW, stride, pad, _tp(inv_smooth),
        _tp(L1p) if R else None, R, _tp(a_codes), _tp(a_scales), _tp(D) if R else None,
        _stream(stream)), "svdq_quantize_act_lowrank_down_conv")


def conv2d(X, KH: int, KW: int, stride: int, pad: int, inv_smooth, L1p, L2t, R: int, w_codes,
           w_scales, bias, Y, ws, stream=None, activation=None):
    """The whole convolution: Y (batch x OH x OW x N, contiguous) from the NHWC image X."""
    B, H, W, Cc, OH, OW, M, K = _conv_shape(X, KH, KW, stride, pad)
    N = _conv_out(Y, B, OH, OW)
    _down(K, R, inv_smooth, L1p)
    _weights(N, K, R, w_codes, w_scales, L2t)
    _bias(bias, N)
    _buf("ws", ws, _BYTES + _HALF + _F32, min_bytes=linear_workspace_bytes(M, K, R))
    _on_gpu(X, inv_smooth, L1p if R else None, L2t if R else None, w_codes, w_scales, bias, Y, ws)
    check(lib.svdq_conv2d(_tp(X), _dt(X), B, H, W, Cc, KH, KW, stride, pad, _tp(inv_smooth),
                          _tp(L1p) if R else None, _tp(L2t) if R else None, R, _tp(w_codes),
                          _tp(w_scales), _tp(bias), _tp(Y), _dt(Y), N, _tp(ws),
                          ws.numel() * ws.element_size(), _act(activation), _stream(stream)),
          "svdq_conv2d")


def quantize_act_lowrank_down_conv_tiled(X, KH: int, KW: int, stride: int, pad: int, inv_smooth,
                                         L1p, R: int, a_ops_t, a_scales_t, D_t, stream=None):
    """K1 on the patch matrix of the NHWC image X, writing the tiled INT4 layouts."""
    B, H, W, Cc, OH, OW, M, K = _conv_shape(X, KH, KW, stride, pad)
    _down(K, R, inv_smooth, L1p)
    _act_side_tiled(M, K, R, a_ops_t, a_scales_t, D_t)
    _on_gpu(X, inv_smooth, L1p if R else None, a_ops_t, a_scales_t, D_t if R else None)
    check(lib.svdq_quantize_act_lowrank_down_conv_tiled(
        _tp(X), _dt(X), B, H, W, Cc, KH, KW, stride, pad, _tp(inv_smooth),
        _tp(L1p) if R else None, R, _tp(a_ops_t), _tp(a_scales_t), _tp(D_t) if R else None,
        _stream(stream)), "svdq_quantize_act_lowrank_down_conv_tiled")


def conv2d_tiled(X, KH: int, KW: int, stride: int, pad: int, inv_smooth, L1p, L2t, R: int,
                 w_codes_t, w_scales_t, bias, Y, ws, stream=None, activation=None):
    """The whole convolution on the tiled INT4 path (weights from pack_w4a4_tiles)."""
    B, H, W, Cc, OH, OW, M, K = _conv_shape(X, KH, KW, stride, pad)
    N = _conv_out(Y, B, OH, OW)
    _down(K, R, inv_smooth, L1p)
    _weights_tiled(N, K, R, w_codes_t, w_scales_t, L2t)
    _bias(bias, N)
    _buf("ws", ws, _BYTES + _HALF + _F32, min_bytes=linear_tiled_workspace_bytes(M, K, R))
    _on_gpu(X, inv_smooth, L1p if R else None, L2t if R else None, w_codes_t, w_scales_t, bias, Y,
            ws)
    check(lib.svdq_conv2d_tiled(_tp(X), _dt(X), B, H, W, Cc, KH, KW, stride, pad, _tp(inv_smooth),
                                _tp(L1p) if R else None, _tp(L2t) if R else None, R,
                                _tp(w_codes_t), _tp(w_scales_t), _tp(bias), _tp(Y), _dt(Y), N,
                                _tp(ws), ws.numel() * ws.element_size(), _act(activation),
                                _stream(stream)),
          "svdq_conv2d_tiled")


def quantize_act_lowrank_down_conv_mx(X, KH: int, KW: int, stride: int, pad: int, inv_smooth,
                                      L1p, R: int, a_codes_t, a_exps_t, D, stream=None):
    """K1-MX on the patch matrix of the NHWC image X: tiled codes and exponents, D."""
    B, H, W, Cc, OH, OW, M, K = _conv_shape(X, KH, KW, stride, pad)
    _down(K, R, inv_smooth, L1p)
    _act_side(M, K, R, a_codes_t, a_exps_t, D, mx=True)
    _on_gpu(X, inv_smooth, L1p if R else None, a_codes_t, a_exps_t, D if R else None)
    check(lib.svdq_quantize_act_lowrank_down_conv_mx(
        _tp(X), _dt(X), B, H, W, Cc, KH, KW, stride, pad, _tp(inv_smooth),
        _tp(L1p) if R else None, R, _tp(a_codes_t), _tp(a_exps_t), _tp(D) if R else None,
        _stream(stream)), "svdq_quantize_act_lowrank_down_conv_mx")


def conv2d_mx(X, KH: int, KW: int, stride: int, pad: int, inv_smooth, L1p, L2t, R: int,
              w_codes_t, w_exps_t, bias, Y, ws, stream=None, activation=None):
    """The whole convolution in MXFP4 (tiled weights): Y (batch x OH x OW x N) from X."""
    B, H, W, Cc, OH, OW, M, K = _conv_shape(X, KH, KW, stride, pad)
    N = _conv_out(Y, B, OH, OW)
    _down(K, R, inv_smooth, L1p)
    _weights(N, K, R, w_codes_t, w_exps_t, L2t, mx=True)
    _bias(bias, N)
    _buf("ws", ws, _BYTES + _HALF + _F32, min_bytes=linear_mx_workspace_bytes(M, K, R))
    _on_gpu(X, inv_smooth, L1p if R else None, L2t if R else None, w_codes_t, w_exps_t, bias, Y,
            ws)
    check(lib.svdq_conv2d_mx(_tp(X), _dt(X), B, H, W, Cc, KH, KW, stride, pad, _tp(inv_smooth),
                             _tp(L1p) if R else None, _tp(L2t) if R else None, R, _tp(w_codes_t),
                             _tp(w_exps_t), _tp(bias), _tp(Y), _dt(Y), N, _tp(ws),
                             ws.numel() * ws.element_size(), _act(activation), _stream(stream)),
          "svdq_conv2d_mx")


def debug_group_partials(a_codes, w_codes, M: int, N: int, K: int, row0: int, rows: int, P,
                         stream=None):
    G = _groups(K)
    _buf("a_codes", a_codes, _BYTES, min_bytes=M * K // 2)
    _buf("w_codes", w_codes, _BYTES, min_bytes=N * K // 2)
    _buf("P", P, ("int32",), min_bytes=4 * max(rows, 0) * N * G)
    _on_gpu(a_codes, w_codes, P)
    check(lib.svdq_debug_group_partials(_tp(a_codes), _tp(w_codes), M, N, K, GROUP, row0, rows,
                                        _tp(P), _stream(stream)), "svdq_debug_group_partials")


def clock_rates():
    """(wall counter rate, peak shader clock), both in kHz, of the current device."""
    import ctypes as C
    w, c = C.c_int32(0), C.c_int32(0)
    check(lib.svdq_clock_rates(C.byref(w), C.byref(c)), "svdq_clock_rates")
    return int(w.value), int(c.value)


def clock_probe(samples, stop, interval_ticks: int, stream=None):
    """Shader-clock sampler (one wave) on `stream`; samples: int64 device tensor of
    1 + 2*n entries, stop: int32 device tensor (zero), see svdq_clock_probe."""
    _buf("samples", samples, ("int64", "uint64"), min_bytes=24)
    _buf("stop", stop, ("int32",), min_bytes=4)
    _on_gpu(samples, stop)
    n = (samples.numel() - 1) // 2
    check(lib.svdq_clock_probe(_tp(samples), n, int(interval_ticks), _tp(stop), _stream(stream)),
          "svdq_clock_probe")


def clock_mark(stamp, stop=None, stream=None):
    """Store the wall counter at stamp[0] and, if given, set stop to end a probe."""
    _buf("stamp", stamp, ("int64", "uint64"), min_bytes=8)
    if stop is not None:
        _buf("stop", stop, ("int32",), min_bytes=4)
    _on_gpu(stamp, stop)
    check(lib.svdq_clock_mark(_tp(stamp), _tp(stop), _stream(stream)), "svdq_clock_mark")


def gelu_tanh_f16(x, y, stream=None):
    _buf("x", x, ("float16",))
    _buf("y", y, ("float16",), min_bytes=2 * x.numel())
    _on_gpu(x, y)
    check(lib.svdq_gelu_tanh_f16(_tp(x), _tp(y), x.numel(), _stream(stream)), "svdq_gelu_tanh_f16")


class Linear:
    """One prepared SVDQuant layer resident on a device.

    ``Linear(prep, bias)(X)`` runs K1 then K2 (their MXFP4 versions for a
    prep of fmt "mxfp4"; with ``tiled=True`` an INT4 prep runs the tiled path,
    svdq_linear_tiled) on the current stream and
    returns Y (M x N, ``out_dtype``), optionally through the fused activation
    (``"gelu_tanh"``). The workspace is kept between calls and grown when a
    larger M arrives."""

    def __init__(self, prep: Prepared, bias: Optional[np.ndarray] = None, device="cuda",
                 out_dtype=None, activation=None, tiled: bool = False):
        torch = _torch()
        self.K, self.N, self.R = prep.K, prep.N, prep.rank
        dev = torch.device(device)
        self.inv_smooth = torch.from_numpy(prep.inv_smooth).to(dev)
        self.L1p = torch.from_numpy(prep.L1p.view(np.int16)).to(dev) if self.R else None
        self.L2t = torch.from_numpy(prep.L2t.view(np.int16)).to(dev) if self.R else None
        self.fmt = prep.fmt
        self.tiled = bool(tiled) and self.fmt == "int4"
        if self.tiled:
            ct, st = pack_w4a4_tiles(prep.w_codes, prep.w_scales, prep.K)
            self.w_codes = torch.from_numpy(ct).to(dev)
            self.w_scales = torch.from_numpy(st).to(dev)
        elif self.fmt == "w4a16":
            ct, st = pack_w4a16_tiles(prep.w_codes, prep.w_scales, prep.K)
            self.w_codes = torch.from_numpy(ct).to(dev)
            self.w_scales = torch.from_numpy(st.view(np.int16)).to(dev)
        elif self.fmt == "mxfp4":
            ct, et = pack_mx_tiles(prep.w_codes, prep.w_scales, prep.K)
            self.w_codes = torch.from_numpy(ct).to(dev)
            self.w_scales = torch.from_numpy(et).to(dev)
        else:
            self.w_codes = torch.from_numpy(prep.w_codes).to(dev)
            self.w_scales = torch.from_numpy(prep.w_scales.view(np.int16)).to(dev)
        self.bias = None if bias is None else torch.from_numpy(_c(bias, np.float32)).to(dev)
        self.out_dtype = out_dtype
        self.activation = activation
        self.device = dev
        self.ws = None

    def workspace(self, M: int):
        torch = _torch()
        if self.fmt == "w4a16":
            need = w4a16_x_tiled_bytes(M, self.K)
        elif self.fmt == "mxfp4":
            need = linear_mx_workspace_bytes(M, self.K, self.R)
        elif self.tiled:
            # the layer's intermediates, then room for the GEMM's split along K
            need = (linear_tiled_workspace_bytes(M, self.K, self.R)
                    + gemm_tiled_workspace_bytes(M, self.N, self.K))
        else:
            need = linear_workspace_bytes(M, self.K, self.R)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self.ws

    def __call__(self, X, Y=None, stream=None):
        torch = _torch()
        _mat("X", X, None, self.K)
        M = X.shape[0]
        if Y is not None:
            _mat("Y", Y, M, self.N)
        if Y is None:
            Y = torch.empty((M, self.N), dtype=self.out_dtype or X.dtype, device=self.device)
        if self.fmt == "w4a16":
            if self.activation is not None:
                raise ValueError("the weight-only baseline has no fused activation")
            linear_w4a16(X, self.w_codes, self.w_scales, self.bias, Y, self.workspace(M), stream)
            return Y
        run = linear_mx if self.fmt == "mxfp4" else linear_tiled if self.tiled else linear
        run(X, self.inv_smooth, self.L1p, self.L2t, self.R, self.w_codes, self.w_scales,
            self.bias, Y, self.workspace(M), stream, self.activation)
        return Y


class Conv2d:
    """One prepared SVDQuant convolution resident on a device.

    ``prep`` is the INT4 or MXFP4 prep of the K x N weight matrix whose row
    (kh*KW + kw)*C + c is filter tap (kh, kw, c) (a KH x KW x C x N filter
    reshaped). ``Conv2d(prep, KH, KW, stride, pad, bias)(X)`` maps an NHWC
    image to the NHWC output (batch x OH x OW x N); with ``tiled=True`` an INT4
    prep runs the tiled path (svdq_conv2d_tiled)."""

    def __init__(self, prep: Prepared, KH: int, KW: int, stride: int = 1, pad: int = 0,
                 bias: Optional[np.ndarray] = None, device="cuda", out_dtype=None,
                 activation=None, tiled: bool = False):
        if prep.fmt not in ("int4", "mxfp4"):
            raise ValueError("convolutions run in the INT4 and MXFP4 formats")
        if prep.K % (KH * KW) != 0:
            raise ValueError(f"K={prep.K} is not KH*KW*C for a {KH}x{KW} kernel")
        self.lin = Linear(prep, bias, device, out_dtype, activation, tiled=tiled)
        self.KH, self.KW, self.stride, self.pad = KH, KW, stride, pad
        self.C = prep.K // (KH * KW)

    def __call__(self, X, Y=None, stream=None):
        torch = _torch()
        lin = self.lin
        B, H, W, Cc = X.shape
        if Cc != self.C:
            raise ValueError(f"image has {Cc} channels, the filter {self.C}")
        OH = conv_out_size(H, self.KH, self.stride, self.pad)
        OW = conv_out_size(W, self.KW, self.stride, self.pad)
        if Y is None:
            Y = torch.empty((B, OH, OW, lin.N), dtype=lin.out_dtype or X.dtype,
                            device=lin.device)
        ws = lin.workspace(max(B * OH * OW, 1))
        run = conv2d_mx if lin.fmt == "mxfp4" else conv2d_tiled if lin.tiled else conv2d
        run(X, self.KH, self.KW, self.stride, self.pad, lin.inv_smooth, lin.L1p, lin.L2t, lin.R,
            lin.w_codes, lin.w_scales, lin.bias, Y, ws, stream, lin.activation)
        return Y
