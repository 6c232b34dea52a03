"""ctypes binding of libsvdq.so (the C ABI in include/svdq.h).

Argument marshalling only: every computation happens in the library. If the
library has not been built this module raises ImportError; there is no
fallback.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvdq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m bit_post_quantized_smooth_amd.build` "
        "(hipcc for gfx950). There is no CPU fallback.")

# PyTorch-ROCm ships its own HIP runtime with the same soname as the system
# one. Whichever is loaded first serves the whole process, so torch (when
# present) is imported first: its allocations, its streams and our launches
# must all go through the runtime torch was built against.
try:
    import torch  # noqa: F401
except ImportError:
    torch = None

lib = C.CDLL(LIB_PATH)

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DTYPE, ERR_RANK, ERR_WORKSPACE, ERR_HIP, \
    ERR_NO_DEVICE, ERR_INTERNAL, ERR_GROUP, ERR_ACT = range(12)
ACT_NONE, ACT_GELU_TANH = 0, 1
F16, F32 = 1, 2
GROUP = 64
MX_BLOCK = 32
MAX_RANK = 256
NOALLOC_MAX_BYTES = 64 << 20

_p = C.c_void_p
_i64 = C.c_int64
_i32 = C.c_int32
_int = C.c_int

_SIGS = {
    "svdq_abi_version": (_int, []),
    "svdq_status_str": (C.c_char_p, [_int]),
    "svdq_last_error": (C.c_char_p, []),
    "svdq_channel_absmax": (_int, [_p, _int, _i64, _i64, _i64, _p]),
    "svdq_smoothing_factors": (_int, [_p, _p, _i64, _i64, _p]),
    "svdq_prepare_weights": (_int, [_p, _p, _i64, _i64, _i32, _i32, _p, _p, _p, _p, _p, _p]),
    "svdq_concat_lora": (_int, [_p, _p, _i64, _i64, _i32, _p, _p, _p, _i32, C.c_float, _p, _p]),
    "svdq_pack_lowrank_down": (_int, [_p, _i64, _i32, _p]),
    "svdq_pack_lowrank": (_int, [_p, _p, _i64, _i64, _i32, _p, _p]),
    "svdq_quantize_act_lowrank_down": (_int, [_p, _int, _i64, _i64, _i64, _p, _p, _i32, _i32,
                                              _p, _p, _p, _p]),
    "svdq_w4a4_gemm_lowrank_up": (_int, [_p, _p, _p, _p, _p, _p, _i32, _p, _p, _int, _i64, _i64,
                                         _i64, _i64, _i32, _i32, _p]),
    "svdq_linear_workspace_bytes": (C.c_size_t, [_i64, _i64, _i32, _i32]),
    "svdq_linear": (_int, [_p, _int, _i64, _p, _p, _p, _i32, _p, _p, _p, _p, _int, _i64, _i64,
                           _i64, _i64, _i32, _p, C.c_size_t, _i32, _p]),
    "svdq_linear_canonical_workspace_bytes": (C.c_size_t, [_i64, _i64, _i64, _i32, _i32]),
    "svdq_linear_canonical": (_int, [_p, _int, _i64, _p, _p, _p, _i32, _p, _p, _p, _p, _int,
                                     _i64, _i64, _i64, _i64, _i32, _p, C.c_size_t, _i32, _p]),
    "svdq_prepare_weights_mx": (_int, [_p, _p, _i64, _i64, _i32, _p, _p, _p, _p, _p, _p]),
    "svdq_quantize_act_lowrank_down_mx": (_int, [_p, _int, _i64, _i64, _i64, _p, _p, _i32, _p, _p,
                                                 _p, _p, C.c_size_t, _p]),
    "svdq_mx_gemm_lowrank_up": (_int, [_p, _p, _p, _p, _p, _p, _i32, _p, _p, _int, _i64, _i64,
                                       _i64, _i64, _i32, _p]),
    "svdq_linear_noalloc": (_int, [_p, _int, _i64, _p, _p, _p, _i32, _p, _p, _p, _p, _int, _i64,
                                   _i64, _i64, _i64, _i32, _i32, _p]),
    "svdq_int4_act_tiled_bytes": (C.c_size_t, [_i64, _i64]),
    "svdq_int4_act_scales_tiled_bytes": (C.c_size_t, [_i64, _i64]),
    "svdq_int4_d_tiled_bytes": (C.c_size_t, [_i64, _i32]),
    "svdq_int4_w_codes_tiled_bytes": (C.c_size_t, [_i64, _i64]),
    "svdq_int4_w_scales_tiled_bytes": (C.c_size_t, [_i64, _i64]),
    "svdq_pack_w4a4_tiles": (_int, [_p, _p, _i64, _i64, _p, _p]),
    "svdq_quantize_act_workspace_bytes": (C.c_size_t, [_i64, _i64, _i32]),
    "svdq_quantize_act_lowrank_down_tiled": (_int, [_p, _int, _i64, _i64, _i64, _p, _p, _i32,
                                                    _p, _p, _p, _p, C.c_size_t, _p]),
    "svdq_gemm_tiled_workspace_bytes": (C.c_size_t, [_i64, _i64, _i64]),
    "svdq_w4a4_gemm_lowrank_up_tiled": (_int, [_p, _p, _p, _p, _p, _p, _i32, _p, _p, _int, _i64,
                                               _i64, _i64, _i64, _i32, _p, C.c_size_t, _p]),
    "svdq_linear_tiled_workspace_bytes": (C.c_size_t, [_i64, _i64, _i32]),
    "svdq_linear_tiled": (_int, [_p, _int, _i64, _p, _p, _p, _i32, _p, _p, _p, _p, _int, _i64,
                                 _i64, _i64, _i64, _p, C.c_size_t, _i32, _p]),
    "svdq_linear_mx_workspace_bytes": (C.c_size_t, [_i64, _i64, _i32]),
    "svdq_mx_codes_tiled_bytes": (C.c_size_t, [_i64, _i64]),
    "svdq_mx_exps_tiled_bytes": (C.c_size_t, [_i64, _i64]),
    "svdq_pack_mx_tiles": (_int, [_p, _p, _i64, _i64, _p, _p]),
    "svdq_linear_mx": (_int, [_p, _int, _i64, _p, _p, _p, _i32, _p, _p, _p, _p, _int, _i64, _i64,
                              _i64, _i64, _p, C.c_size_t, _i32, _p]),
    "svdq_prepare_weights_w4a16": (_int, [_p, _i64, _i64, _p, _p]),
    "svdq_w4a16_codes_tiled_bytes": (C.c_size_t, [_i64, _i64]),
    "svdq_w4a16_scales_tiled_bytes": (C.c_size_t, [_i64, _i64]),
    "svdq_w4a16_x_tiled_bytes": (C.c_size_t, [_i64, _i64]),
    "svdq_pack_w4a16_tiles": (_int, [_p, _p, _i64, _i64, _p, _p]),
    "svdq_w4a16_tile_activation": (_int, [_p, _int, _i64, _i64, _i64, _p, _p]),
    "svdq_w4a16_gemm": (_int, [_p, _p, _p, _p, _p, _int, _i64, _i64, _i64, _i64, _p]),
    "svdq_linear_w4a16": (_int, [_p, _int, _i64, _p, _p, _p, _p, _int, _i64, _i64, _i64, _i64,
                                 _p, C.c_size_t, _p]),
    "svdq_conv_patch_absmax": (_int, [_p, _int, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _i32,
                                      _p]),
    "svdq_quantize_act_lowrank_down_conv": (_int, [_p, _int, _i64, _i64, _i64, _i64, _i32, _i32,
                                                   _i32, _i32, _p, _p, _i32, _p, _p, _p, _p]),
    "svdq_conv2d": (_int, [_p, _int, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _p, _p, _p,
                           _i32, _p, _p, _p, _p, _int, _i64, _p, C.c_size_t, _i32, _p]),
    "svdq_quantize_act_lowrank_down_conv_tiled": (_int, [_p, _int, _i64, _i64, _i64, _i64, _i32,
                                                         _i32, _i32, _i32, _p, _p, _i32, _p, _p,
                                                         _p, _p]),
    "svdq_conv2d_tiled": (_int, [_p, _int, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _p, _p,
                                 _p, _i32, _p, _p, _p, _p, _int, _i64, _p, C.c_size_t, _i32, _p]),
    "svdq_quantize_act_lowrank_down_conv_mx": (_int, [_p, _int, _i64, _i64, _i64, _i64, _i32, _i32,
                                                      _i32, _i32, _p, _p, _i32, _p, _p, _p, _p]),
    "svdq_conv2d_mx": (_int, [_p, _int, _i64, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _p, _p,
                              _p, _i32, _p, _p, _p, _p, _int, _i64, _p, C.c_size_t, _i32, _p]),
    "svdq_debug_group_partials": (_int, [_p, _p, _i64, _i64, _i64, _i32, _i64, _i64, _p, _p]),
    "svdq_gelu_tanh_f16": (_int, [_p, _p, _i64, _p]),
    "svdq_clock_rates": (_int, [_p, _p]),
    "svdq_clock_probe": (_int, [_p, _i32, _i64, _p, _p]),
    "svdq_clock_mark": (_int, [_p, _p, _p]),
}

for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


class SvdqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.svdq_last_error().decode() or lib.svdq_status_str(status).decode()
        super().__init__(f"{where}: status {status} ({lib.svdq_status_str(status).decode()}): {msg}")


def check(status: int, where: str) -> None:
    if status != OK:
        raise SvdqError(status, where)


def status_str(status: int) -> str:
    return lib.svdq_status_str(status).decode()


def last_error() -> str:
    return lib.svdq_last_error().decode()


def abi_version() -> int:
    return lib.svdq_abi_version()
