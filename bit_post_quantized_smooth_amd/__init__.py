"""SVDQuant W4A4 + low-rank linear layer for AMD Instinct MI355X (gfx950).

The compute lives in libsvdq.so (hand-written HIP kernels behind the C ABI in
include/svdq.h); this package is its thin Python binding. Importing it
without a built library raises ImportError.
"""
from . import _lib  # noqa: F401  (fails loudly when libsvdq.so is missing)
from .api import (Conv2d, Linear, Prepared, channel_absmax, clock_mark, clock_probe,  # noqa: F401
                  clock_rates, concat_lora, int4_act_tiled_bytes, int4_act_scales_tiled_bytes, int4_d_tiled_bytes,
                  int4_w_codes_tiled_bytes, int4_w_scales_tiled_bytes, linear_tiled,
                  linear_tiled_workspace_bytes, pack_w4a4_tiles, quantize_act_lowrank_down_tiled,
                  quantize_act_workspace_bytes, w4a4_gemm_lowrank_up_tiled, gemm_tiled_workspace_bytes,
                  conv2d, conv2d_mx, conv2d_tiled, conv_out_size, conv_patch_absmax, debug_group_partials,
                  gelu_tanh_f16, linear, linear_canonical, linear_canonical_workspace_bytes,
                  linear_mx, linear_mx_workspace_bytes, pack_lowrank,
                  linear_noalloc, linear_workspace_bytes, mx_codes_tiled_bytes, mx_exps_tiled_bytes,
                  mx_gemm_lowrank_up, pack_lowrank_down, pack_mx_tiles, prepare_weights,
                  prepare_weights_mx, prepare_weights_w4a16, pack_w4a16_tiles,
                  quantize_act_lowrank_down, quantize_act_lowrank_down_conv,
                  quantize_act_lowrank_down_conv_mx, quantize_act_lowrank_down_conv_tiled,
                  quantize_act_lowrank_down_mx, smoothing_factors, w4a4_gemm_lowrank_up,
                  w4a16_gemm, w4a16_tile_activation, w4a16_x_tiled_bytes, linear_w4a16)

__all__ = ["Conv2d", "Linear", "Prepared", "channel_absmax", "clock_mark", "clock_probe",
           "clock_rates", "concat_lora", "int4_act_tiled_bytes", "int4_act_scales_tiled_bytes", "int4_d_tiled_bytes",
           "int4_w_codes_tiled_bytes", "int4_w_scales_tiled_bytes", "linear_tiled",
           "linear_tiled_workspace_bytes", "pack_w4a4_tiles", "quantize_act_lowrank_down_tiled",
           "quantize_act_workspace_bytes", "w4a4_gemm_lowrank_up_tiled", "gemm_tiled_workspace_bytes", "conv2d", "conv2d_mx", "conv2d_tiled",
           "conv_out_size", "conv_patch_absmax", "debug_group_partials",
           "gelu_tanh_f16", "linear", "linear_canonical", "linear_canonical_workspace_bytes",
           "linear_mx", "linear_mx_workspace_bytes", "pack_lowrank",
           "linear_noalloc", "linear_workspace_bytes", "mx_codes_tiled_bytes", "mx_exps_tiled_bytes",
           "mx_gemm_lowrank_up", "pack_lowrank_down", "pack_mx_tiles", "prepare_weights",
           "prepare_weights_mx", "quantize_act_lowrank_down", "quantize_act_lowrank_down_conv",
           "quantize_act_lowrank_down_conv_mx", "quantize_act_lowrank_down_conv_tiled",
           "quantize_act_lowrank_down_mx", "smoothing_factors", "w4a4_gemm_lowrank_up",
           "prepare_weights_w4a16", "pack_w4a16_tiles", "w4a16_gemm", "w4a16_tile_activation",
           "w4a16_x_tiled_bytes", "linear_w4a16"]
