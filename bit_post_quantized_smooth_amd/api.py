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


def quantize_act_lowrank_down(X, inv_smooth, L1p, R: int, a_codes, a_scales, D, stream=None):
    M, K = X.shape
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
    M, N = Y.shape
    check(lib.svdq_w4a4_gemm_lowrank_up(_tp(a_codes), _tp(a_scales), _tp(w_codes), _tp(w_scales),
                                        _tp(D) if R else None, _tp(L2t) if R else None, R, _tp(bias),
                                        _tp(Y), _dt(Y), M, N, K, Y.stride(0), GROUP,
                                        _act(activation), _stream(stream)),
          "svdq_w4a4_gemm_lowrank_up")


def linear_workspace_bytes(M: int, K: int, R: int) -> int:
    return int(lib.svdq_linear_workspace_bytes(M, K, R, GROUP))


def linear(X, inv_smooth, L1p, L2t, R: int, w_codes, w_scales, bias, Y, ws, stream=None,
           activation=None):
    M, K = X.shape
    N = Y.shape[1]
    check(lib.svdq_linear(_tp(X), _dt(X), X.stride(0), _tp(inv_smooth), _tp(L1p) if R else None,
                          _tp(L2t) if R else None, R, _tp(w_codes), _tp(w_scales), _tp(bias), _tp(Y),
                          _dt(Y), Y.stride(0), M, K, N, GROUP, _tp(ws), ws.numel() * ws.element_size(),
                          _act(activation), _stream(stream)), "svdq_linear")


def quantize_act_lowrank_down_mx(X, inv_smooth, L1p, R: int, a_codes_t, a_exps_t, D, stream=None):
    """K1-MX; a_codes_t / a_exps_t: device buffers of mx_codes_tiled_bytes(M, K) and
    mx_exps_tiled_bytes(M, K) bytes (tiled layouts)."""
    M, K = X.shape
    check(lib.svdq_quantize_act_lowrank_down_mx(_tp(X), _dt(X), M, K, X.stride(0), _tp(inv_smooth),
                                                _tp(L1p) if R else None, R, _tp(a_codes_t),
                                                _tp(a_exps_t), _tp(D) if R else None,
                                                _stream(stream)),
          "svdq_quantize_act_lowrank_down_mx")


def mx_gemm_lowrank_up(a_codes_t, a_exps_t, w_codes_t, w_exps_t, D, L2t, R: int, bias, Y, K: int,
                       stream=None, activation=None):
    """K2-MX on the tiled activation and weight codes and exponents."""
    M, N = Y.shape
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
    M, K = X.shape
    N = Y.shape[1]
    check(lib.svdq_linear_mx(_tp(X), _dt(X), X.stride(0), _tp(inv_smooth),
                             _tp(L1p) if R else None, _tp(L2t) if R else None, R, _tp(w_codes_t),
                             _tp(w_exps_t), _tp(bias), _tp(Y), _dt(Y), Y.stride(0), M, K, N, _tp(ws),
                             ws.numel() * ws.element_size(), _act(activation), _stream(stream)),
          "svdq_linear_mx")


def w4a16_x_tiled_bytes(M: int, K: int) -> int:
    return int(lib.svdq_w4a16_x_tiled_bytes(M, K))


def w4a16_tile_activation(X, x_t, stream=None):
    """X (fp16 or fp32, M x K) -> x_t (w4a16_x_tiled_bytes(M, K) bytes), the tiled fp16 layout."""
    M, K = X.shape
    check(lib.svdq_w4a16_tile_activation(_tp(X), _dt(X), M, K, X.stride(0), _tp(x_t),
                                         _stream(stream)), "svdq_w4a16_tile_activation")


def w4a16_gemm(x_t, w_codes_t, w_scales_t, bias, Y, K: int, stream=None):
    M, N = Y.shape
    check(lib.svdq_w4a16_gemm(_tp(x_t), _tp(w_codes_t), _tp(w_scales_t), _tp(bias), _tp(Y), _dt(Y),
                              M, N, K, Y.stride(0), _stream(stream)), "svdq_w4a16_gemm")


def linear_w4a16(X, w_codes_t, w_scales_t, bias, Y, ws, stream=None):
    """The weight-only baseline layer (tiling of X into ws, then the GEMM)."""
    M, K = X.shape
    N = Y.shape[1]
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


def quantize_act_lowrank_down_conv(X, KH: int, KW: int, stride: int, pad: int, inv_smooth, L1p,
                                   R: int, a_codes, a_scales, D, stream=None):
    """K1 on the patch matrix of the NHWC image X (batch x H x W x C, contiguous)."""
    B, H, W, Cc = X.shape
    check(lib.svdq_quantize_act_lowrank_down_conv(
        _tp(X), _dt(X), B, H, W, Cc, KH, KW, stride, pad, _tp(inv_smooth),
        _tp(L1p) if R else None, R, _tp(a_codes), _tp(a_scales), _tp(D) if R else None,
        _stream(stream)), "svdq_quantize_act_lowrank_down_conv")


def conv2d(X, KH: int, KW: int, stride: int, pad: int, inv_smooth, L1p, L2t, R: int, w_codes,
           w_scales, bias, Y, ws, stream=None, activation=None):
    """The whole convolution: Y (batch x OH x OW x N, contiguous) from the NHWC image X."""
    B, H, W, Cc = X.shape
    N = Y.shape[-1]
    check(lib.svdq_conv2d(_tp(X), _dt(X), B, H, W, Cc, KH, KW, stride, pad, _tp(inv_smooth),
                          _tp(L1p) if R else None, _tp(L2t) if R else None, R, _tp(w_codes),
                          _tp(w_scales), _tp(bias), _tp(Y), _dt(Y), N, _tp(ws),
                          ws.numel() * ws.element_size(), _act(activation), _stream(stream)),
          "svdq_conv2d")


def quantize_act_lowrank_down_conv_mx(X, KH: int, KW: int, stride: int, pad: int, inv_smooth,
                                      L1p, R: int, a_codes_t, a_exps_t, D, stream=None):
    """K1-MX on the patch matrix of the NHWC image X: tiled codes and exponents, D."""
    B, H, W, Cc = X.shape
    check(lib.svdq_quantize_act_lowrank_down_conv_mx(
        _tp(X), _dt(X), B, H, W, Cc, KH, KW, stride, pad, _tp(inv_smooth),
        _tp(L1p) if R else None, R, _tp(a_codes_t), _tp(a_exps_t), _tp(D) if R else None,
        _stream(stream)), "svdq_quantize_act_lowrank_down_conv_mx")


def conv2d_mx(X, KH: int, KW: int, stride: int, pad: int, inv_smooth, L1p, L2t, R: int,
              w_codes_t, w_exps_t, bias, Y, ws, stream=None, activation=None):
    """The whole convolution in MXFP4 (tiled weights): Y (batch x OH x OW x N) from X."""
    B, H, W, Cc = X.shape
    N = Y.shape[-1]
    check(lib.svdq_conv2d_mx(_tp(X), _dt(X), B, H, W, Cc, KH, KW, stride, pad, _tp(inv_smooth),
                             _tp(L1p) if R else None, _tp(L2t) if R else None, R, _tp(w_codes_t),
                             _tp(w_exps_t), _tp(bias), _tp(Y), _dt(Y), N, _tp(ws),
                             ws.numel() * ws.element_size(), _act(activation), _stream(stream)),
          "svdq_conv2d_mx")


def debug_group_partials(a_codes, w_codes, M: int, N: int, K: int, row0: int, rows: int, P,
                         stream=None):
    check(lib.svdq_debug_group_partials(_tp(a_codes), _tp(w_codes), M, N, K, GROUP, row0, rows,
                                        _tp(P), _stream(stream)), "svdq_debug_group_partials")


def gelu_tanh_f16(x, y, stream=None):
    check(lib.svdq_gelu_tanh_f16(_tp(x), _tp(y), x.numel(), _stream(stream)), "svdq_gelu_tanh_f16")


class Linear:
    """One prepared SVDQuant layer resident on a device.

    ``Linear(prep, bias)(X)`` runs K1 then K2 (their MXFP4 versions for a
    prep of fmt "mxfp4") on the current stream and
    returns Y (M x N, ``out_dtype``), optionally through the fused activation
    (``"gelu_tanh"``). The workspace is kept between calls and grown when a
    larger M arrives."""

    def __init__(self, prep: Prepared, bias: Optional[np.ndarray] = None, device="cuda",
                 out_dtype=None, activation=None):
        torch = _torch()
        self.K, self.N, self.R = prep.K, prep.N, prep.rank
        dev = torch.device(device)
        self.inv_smooth = torch.from_numpy(prep.inv_smooth).to(dev)
        self.L1p = torch.from_numpy(prep.L1p.view(np.int16)).to(dev) if self.R else None
        self.L2t = torch.from_numpy(prep.L2t.view(np.int16)).to(dev) if self.R else None
        self.fmt = prep.fmt
        if self.fmt == "w4a16":
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
        else:
            need = linear_workspace_bytes(M, self.K, self.R)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self.ws

    def __call__(self, X, Y=None, stream=None):
        torch = _torch()
        M = X.shape[0]
        if Y is None:
            Y = torch.empty((M, self.N), dtype=self.out_dtype or X.dtype, device=self.device)
        if self.fmt == "w4a16":
            if self.activation is not None:
                raise ValueError("the weight-only baseline has no fused activation")
            linear_w4a16(X, self.w_codes, self.w_scales, self.bias, Y, self.workspace(M), stream)
            return Y
        run = linear_mx if self.fmt == "mxfp4" else linear
        run(X, self.inv_smooth, self.L1p, self.L2t, self.R, self.w_codes, self.w_scales,
            self.bias, Y, self.workspace(M), stream, self.activation)
        return Y


class Conv2d:
    """One prepared SVDQuant convolution resident on a device.

    ``prep`` is the INT4 or MXFP4 prep of the K x N weight matrix whose row
    (kh*KW + kw)*C + c is filter tap (kh, kw, c) (a KH x KW x C x N filter
    reshaped). ``Conv2d(prep, KH, KW, stride, pad, bias)(X)`` maps an NHWC
    image to the NHWC output (batch x OH x OW x N)."""

    def __init__(self, prep: Prepared, KH: int, KW: int, stride: int = 1, pad: int = 0,
                 bias: Optional[np.ndarray] = None, device="cuda", out_dtype=None,
                 activation=None):
        if prep.fmt not in ("int4", "mxfp4"):
            raise ValueError("convolutions run in the INT4 and MXFP4 formats")
        if prep.K % (KH * KW) != 0:
            raise ValueError(f"K={prep.K} is not KH*KW*C for a {KH}x{KW} kernel")
        self.lin = Linear(prep, bias, device, out_dtype, activation)
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
        run = conv2d_mx if lin.fmt == "mxfp4" else conv2d
        run(X, self.KH, self.KW, self.stride, self.pad, lin.inv_smooth, lin.L1p, lin.L2t, lin.R,
            lin.w_codes, lin.w_scales, lin.bias, Y, ws, stream, lin.activation)
        return Y
