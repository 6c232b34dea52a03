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

// a_meta: fp16 group scales (mx = false) or E8M0 block exponents (mx = true).
// conv: null for a linear layer; else X is the NHWC image and M, K are the
// patch matrix's.
hipError_t launch_k1(const void* X, bool x_f16, int64_t M, int64_t K, int64_t ldx,
                     const float* inv_smooth, const uint16_t* L1p, int R, uint8_t* a_codes,
                     void* a_meta, bool mx, float* D, hipStream_t stream,
                     const ConvGeom* conv = nullptr);

hipError_t launch_k2(const uint8_t* a_codes, const uint16_t* a_scales, const uint8_t* w_codes,
                     const uint16_t* w_scales, const float* D, const uint16_t* L2t, int R,
                     const float* bias, void* Y, bool y_f16, int64_t M, int64_t N, int64_t K,
                     int64_t ldy, bool gelu, hipStream_t stream);

hipError_t launch_k2_mx(const uint8_t* a_codes, const uint8_t* a_e8m0, const uint8_t* w_codes,
                        const uint8_t* w_e8m0, const float* D, const uint16_t* L2t, int R,
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

}  // namespace svdq
