// Device-side helpers shared by the gfx950 kernels of libsvdq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kGroup = 64;          // input channels per quantization group
constexpr int kGroupBytes = 32;     // packed 4-bit codes per group

// Bit pattern of 1.5 * 2^23. An int32 accumulator seeded with it and given an
// integer sum s with |s| < 2^22 reads back as the float 12582912 + s exactly,
// which saves the int -> float conversion in the per-group rescale.
constexpr int kMagicSeed = 0x4B400000;
constexpr float kMagicF = 12582912.0f;

// Two's-complement nibbles -> int8 lanes holding 16*q. For a dword w with
// codes c0..c7 (c0 in the low nibble): hi holds 16*c1, 16*c3, 16*c5, 16*c7 and
// lo holds 16*c0, 16*c2, 16*c4, 16*c6, one per byte. Both matrix-core operands
// are widened the same way, so every product carries a factor 256 and the
// order of codes inside the K block is the same on both sides.
__device__ __forceinline__ void unpack_nibbles_x16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  hi = w & 0xF0F0F0F0u;
  lo = (w << 4) & 0xF0F0F0F0u;
}

// 8 packed bytes (16 codes) -> one 16-byte int8 operand for
// v_mfma_i32_16x16x64_i8.
__device__ __forceinline__ v4i widen_codes(uint2 p) {
  uint32_t a0, a1, b0, b1;
  unpack_nibbles_x16(p.x, a0, a1);
  unpack_nibbles_x16(p.y, b0, b1);
  v4i r;
  r[0] = static_cast<int>(a0);
  r[1] = static_cast<int>(a1);
  r[2] = static_cast<int>(b0);
  r[3] = static_cast<int>(b1);
  return r;
}

__device__ __forceinline__ v4i mfma_i8_16x16x64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_f16_16x16x32(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Reinterpret an int32 as fp32. Takes the value (not a vector element
// lvalue): clang lowers __builtin_bit_cast of an ext_vector element as if it
// were element 0, so callers copy the element into a scalar first.
__device__ __forceinline__ float as_float(int v) { return __builtin_bit_cast(float, v); }

__device__ __forceinline__ float h2f(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));   // v_cvt_f16_f32, RNE
}

// GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) in fp32.
// 0.5 x (1 + tanh(u)) written as x / (1 + exp(-2u)) (the same function:
// 0.5 (1 + tanh(u)) is the logistic function of 2u). The second form keeps full
// relative accuracy for large negative x, where 1 + tanh(u) cancels in fp32.
__device__ __forceinline__ float gelu_tanh_f32(float x) {
  const float c2 = 1.5957691216057308f;    // 2 sqrt(2/pi)
  const float u2 = c2 * (x + 0.044715f * x * x * x);
  return x / (1.0f + expf(-u2));
}

}  // namespace svdq
