// Host-side launchers of the gfx950 kernels (called by the C ABI layer after
// it has validated every argument).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

// A KH x KW convolution over an NHWC image (batch x H x W x C), run by K1 as
// the linear layer on its patch matrix: row (b, oh, ow), column
// (kh*KW + kw)*C + c (zero outside the image). C % 64 == 0, so a 64-channel
// group lies within one tap.
struct ConvGeom {
  int32_t H, W, C, KH, KW, stride, pad, OH, OW;
};

// Resident workgroup slots of the current device (2 per compute unit).
int resident_slots();

// Output format of the pre-kernel: canonical INT4 codes and fp16 scales;
// MXFP4 tiled codes and E8M0 exponents; INT4 operand tiles and fp32 scale
// pairs for the tiled GEMM (K2T). a_codes / a_meta are the codes / the scales,
// exponents or scale pairs of that format.
enum K1Fmt { kK1Int4 = 0, kK1Mx = 1, kK1Int4Tiled = 2 };

// conv: null for a linear layer; else X is the NHWC image and M, K are the
// patch matrix's. part: null, or k1_split_bytes(M, K, R, fmt, conv) bytes
// (16-byte aligned) for the partial D tiles of a split pre-kernel; without
// it a shape that would split runs unsplit (ranks above 0).
hipError_t launch_k1(const void* X, bool x_f16, int64_t M, int64_t K, int64_t ldx,
                     const float* inv_smooth, const uint16_t* L1p, int R, uint8_t* a_codes,
                     void* a_meta, int fmt, float* D, hipStream_t stream,
                     const ConvGeom* conv = nullptr, float* part = nullptr);

// Slices of the groups per row tile that the pre-kernel uses for this shape
// on the current device (1: not split), and the bytes its partial D tiles
// need (0 when not split or R = 0).
int k1_slices(int64_t M, int64_t K, int R, int fmt, bool conv);
size_t k1_split_bytes(int64_t M, int64_t K, int R, int fmt, bool conv);

hipError_t launch_k2(const uint8_t* a_codes, const uint16_t* a_scales, const uint8_t* w_codes,
                     const uint16_t* w_scales, const float* D, const uint16_t* L2t, int R,
                     const float* bias, void* Y, bool y_f16, int64_t M, int64_t N, int64_t K,
                     int64_t ldy, bool gelu, hipStream_t stream);

// K2T on the tiled INT4 layouts (svdq.h): a_ops / a_scales from the
// pre-kernel's tiled instance, the weight codes and scale pairs from
// svdq_pack_w4a4_tiles.
// part: null, or k2t_split_bytes(M, N, K) bytes (16-byte aligned) for the
// fp32 partial tiles of the split-along-K kernel; without it every shape runs
// unsplit.
hipError_t launch_k2t(const uint8_t* a_ops, const float* a_scales, const uint8_t* w_codes_t,
                      const float* w_scales_t, const uint16_t* Dt, const uint16_t* L2t, int R,
                      const float* bias, void* Y, bool y_f16, int64_t M, int64_t N, int64_t K,
                      int64_t ldy, bool gelu, hipStream_t stream, float* part = nullptr);

// Slices along K that K2T uses for this shape on the current device (1: not
// split) and the bytes of its partial tiles (0 when not split).
int k2t_ksplit(int64_t M, int64_t N, int64_t K);
size_t k2t_split_bytes(int64_t M, int64_t N, int64_t K);

hipError_t launch_k2_mx(const uint8_t* a_codes, const uint8_t* a_e8m0, const uint8_t* w_codes,
                        const uint8_t* w_e8m0, const uint16_t* Dt, const uint16_t* L2t, int R,
                        const float* bias, void* Y, bool y_f16, int64_t M, int64_t N, int64_t K,
                        int64_t ldy, bool gelu, hipStream_t stream);

hipError_t launch_w4a16_tile_x(const void* X, bool x_f16, int64_t M, int64_t K, int64_t ldx,
                               uint16_t* x_t, hipStream_t stream);

hipError_t launch_w4a16_gemm(const uint16_t* x_t, const uint8_t* w_codes_t,
                             const uint16_t* w_scales_t, const float* bias, void* Y, bool y_f16,
                             int64_t M, int64_t N, int64_t K, int64_t ldy, hipStream_t stream);

hipError_t launch_debug_partials(const uint8_t* a_codes, const uint8_t* w_codes, int64_t M,
                                 int64_t N, int64_t K, int64_t row0, int64_t rows, int32_t* P,
                                 hipStream_t stream);

hipError_t launch_gelu_f16(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t stream);

// The canonical low-rank factors L1 (K x R) and L2 (R x N) -> L1p and L2t
// (see lowrank_pack.hip).
hipError_t launch_pack_lowrank(const uint16_t* L1, const uint16_t* L2, int64_t K, int64_t N,
                               int R, uint16_t* L1p, uint16_t* L2t, hipStream_t stream);

// Measurement utility: shader-clock samples (see clock_probe.hip).
hipError_t launch_clock_probe(uint64_t* samples, int32_t max_samples, int64_t interval,
                              const int32_t* stop, hipStream_t stream);
hipError_t launch_clock_mark(uint64_t* stamp, int32_t* stop, hipStream_t stream);

}  // namespace svdq
