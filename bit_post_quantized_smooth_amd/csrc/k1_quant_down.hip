// K1: the fused pre-kernel of the SVDQuant linear layer (gfx950).
//
// One pass over X does everything the low-bit and low-rank branches need
// from the activation (SVDQuant abstract: running the low-rank branch on its
// own moves the activation again and eats the speedup, so the engine fuses
// it with the low-bit kernels; chattools.cn overview, section
// "SVDQuant的技术原理", Nunchaku item: fusion cuts memory traffic and launches):
//   Xhat = fp32(x) * inv_smooth[k]               (smoothing)
//   per row and group of 64: absmax -> fp16 scale -> 4-bit codes (quantizer)
//   D += fp16(Xhat) . L1                          (down-projection, fp16 MFMA)
//
// Work split: a workgroup owns 16 rows; its waves (8, or 4 at high rank) take the 64-channel groups
// round-robin, so consecutive groups of a row are in flight in neighbouring
// waves and each wave's loads are 16 rows x 128 contiguous bytes. Lane l
// handles row l%16 and the 16 channels 16*(l/16) .. +15 of the group: these
// 16 values are both its quantizer input and, rounded to fp16, its operand
// pieces for v_mfma_f32_16x16x32_f16 (the matching L1 values come from the
// same channels, so the two operands agree on the summation order). The
// per-wave partial D tiles are summed in LDS in a fixed order.
//
// Latency hiding: each wave keeps a ring of NB groups in registers; group i is
// quantized while groups i+1 .. i+NB-1 are in flight, and its slot is then
// refilled with group i+NB. Every load is unconditional (rows past M and
// groups past the wave's last are clamped to valid addresses and their
// results discarded), so the compiler can count outstanding loads exactly and
// never waits for more than the one group it needs.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "device_launch.hpp"

namespace svdq {

// Raw X data of one lane for one group: 16 consecutive values.
template <typename XT>
struct Raw;
template <>
struct Raw<_Float16> {
  uint4 v[2];
};
template <>
struct Raw<float> {
  float4 v[4];
};

template <typename XT>
__device__ __forceinline__ void load_raw(Raw<XT>& r, const XT* p);

template <>
__device__ __forceinline__ void load_raw<_Float16>(Raw<_Float16>& r, const _Float16* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  r.v[0] = q[0];
  r.v[1] = q[1];
}

template <>
__device__ __forceinline__ void load_raw<float>(Raw<float>& r, const float* p) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) r.v[i] = q[i];
}

// xh[i] = fp32(x[i]) * inv[i], rounded once to fp32. For fp16 input this is
// one mixed-precision FMA per value (the fp16 -> fp32 widening is exact, the
// product is rounded once; adding -0 keeps the sign of a zero product).
__device__ __forceinline__ void smooth16(const Raw<_Float16>& r, const float4* inv, float* xh) {
  const uint32_t w[8] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w,
                         r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
  const float iv[16] = {inv[0].x, inv[0].y, inv[0].z, inv[0].w, inv[1].x, inv[1].y,
                        inv[1].z, inv[1].w, inv[2].x, inv[2].y, inv[2].z, inv[2].w,
                        inv[3].x, inv[3].y, inv[3].z, inv[3].w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const _Float16 lo = __builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] & 0xFFFFu));
    const _Float16 hi = __builtin_bit_cast(_Float16, static_cast<uint16_t>(w[i] >> 16));
    xh[2 * i] = __builtin_fmaf(static_cast<float>(lo), iv[2 * i], -0.0f);
    xh[2 * i + 1] = __builtin_fmaf(static_cast<float>(hi), iv[2 * i + 1], -0.0f);
  }
}

__device__ __forceinline__ void smooth16(const Raw<float>& r, const float4* inv, float* xh) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xh[4 * i] = r.v[i].x * inv[i].x;
    xh[4 * i + 1] = r.v[i].y * inv[i].y;
    xh[4 * i + 2] = r.v[i].z * inv[i].z;
    xh[4 * i + 3] = r.v[i].w * inv[i].w;
  }
}

// L1 slices travel in the ring up to rank 128; above that they would not fit
// in registers next to the accumulators and are loaded just before use.
template <int NCB>
constexpr int ring_l1_blocks() { return NCB <= 8 ? NCB : 0; }

// Everything one lane reads for one group: its 16 X values, the 16 matching
// smoothing factors and, per column block of D, the 16 matching L1 values.
template <typename XT, int NCB>
struct GroupIn {
  Raw<XT> x;
  float4 inv[4];
  v8h l1[ring_l1_blocks<NCB>() > 0 ? ring_l1_blocks<NCB>() : 1][2];
};

// Waves per workgroup: 8 while the partial-D tiles of all waves fit in LDS
// next to a second resident workgroup, else 4.
template <int NCB>
constexpr int k1_waves() { return NCB <= 4 ? 8 : 4; }

template <typename XT, int NCB, int NB>
__global__ __launch_bounds__(64 * k1_waves<NCB>(), 2) void k1_quant_down_kernel(
    const XT* __restrict__ X, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ inv_smooth, const uint16_t* __restrict__ L1t, int R,
    uint8_t* __restrict__ a_codes, uint16_t* __restrict__ a_scales, float* __restrict__ D) {
#pragma clang fp contract(off)
  constexpr int K1_WAVES = k1_waves<NCB>();
  __shared__ float dpart[K1_WAVES][16][NCB > 0 ? NCB * 16 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rl = lane & 15, q = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t row = row0 + rl;
  const bool rvalid = row < M;
  const int64_t lrow = rvalid ? row : M - 1;      // clamped row for loads
  const int64_t G = K / kGroup;
  // this wave's groups are wave, wave+4, ...: n_mine of them
  const int64_t n_mine = (G > wave) ? (G - wave + K1_WAVES - 1) / K1_WAVES : 0;

  const XT* xrow = X + lrow * ldx + q * 16;
  const float* invq = inv_smooth + q * 16;
  const uint16_t* l1q = L1t + static_cast<int64_t>(rl) * K + q * 16;

  auto load_group = [&](GroupIn<XT, NCB>& in, int64_t i) {
    int64_t g = wave + K1_WAVES * i;
    g = g < G ? g : G - 1;
    const int64_t k0 = g * kGroup;
    load_raw<XT>(in.x, xrow + k0);
    const float4* ip = reinterpret_cast<const float4*>(invq + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j) in.inv[j] = ip[j];
    if constexpr (ring_l1_blocks<NCB>() > 0) {
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const v8h* lp = reinterpret_cast<const v8h*>(l1q + static_cast<int64_t>(c * 16) * K + k0);
        in.l1[c][0] = lp[0];
        in.l1[c][1] = lp[1];
      }
    }
  };

  v4f acc[NCB > 0 ? NCB : 1];
#pragma unroll
  for (int c = 0; c < (NCB > 0 ? NCB : 1); ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};

  GroupIn<XT, NCB> ring[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) load_group(ring[b], b);

  for (int64_t i0 = 0; i0 < n_mine; i0 += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t i = i0 + b;
      if (i < n_mine) {
        const int64_t g = wave + K1_WAVES * i;
        float xh[16];
        smooth16(ring[b].x, ring[b].inv, xh);
        // group absmax over this lane's 16 values, then across the 4 lanes of the row
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(xh[j]));
        a = fmaxf(a, __shfl_xor(a, 16));
        a = fmaxf(a, __shfl_xor(a, 32));
        const float s32 = fminf(a / 7.0f, 65504.0f);      // correctly rounded division
        const uint16_t s16 = f2h(s32);
        const float sf = h2f(s16);
        const float inv = (sf == 0.f) ? 0.f : 1.0f / sf;
        // code = clamp(rint(xh * inv), -7, 7): clamping first gives the same
        // result, and adding 1.5 * 2^23 rounds half-to-even to an integer whose
        // low 4 bits are its two's-complement nibble.
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float c = __builtin_amdgcn_fmed3f(xh[j] * inv, -7.f, 7.f);
          const uint32_t bits = __builtin_bit_cast(uint32_t, c + kMagicF);
          packed[j >> 3] |= (bits & 0xFu) << (4 * (j & 7));
        }
        if (rvalid) {
          *reinterpret_cast<uint2*>(a_codes + row * (K / 2) + g * kGroupBytes + q * 8) =
              make_uint2(packed[0], packed[1]);
          if (q == 0) a_scales[row * G + g] = s16;
        }
        if constexpr (NCB > 0) {
          v8h x0, x1;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            x0[j] = static_cast<_Float16>(xh[j]);
            x1[j] = static_cast<_Float16>(xh[8 + j]);
          }
          if constexpr (ring_l1_blocks<NCB>() > 0) {
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
              acc[c] = mfma_f16_16x16x32(x0, ring[b].l1[c][0], acc[c]);
              acc[c] = mfma_f16_16x16x32(x1, ring[b].l1[c][1], acc[c]);
            }
          } else {
#pragma unroll
            for (int c = 0; c < NCB; ++c) {
              const v8h* lp =
                  reinterpret_cast<const v8h*>(l1q + static_cast<int64_t>(c * 16) * K + g * kGroup);
              acc[c] = mfma_f16_16x16x32(x0, lp[0], acc[c]);
              acc[c] = mfma_f16_16x16x32(x1, lp[1], acc[c]);
            }
          }
        }
      }
      load_group(ring[b], i + NB);
    }
  }

  if constexpr (NCB > 0) {
    // partial D of this wave -> LDS; lane holds rows 4q+i of column c*16+rl
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) dpart[wave][4 * q + j][c * 16 + rl] = acc[c][j];
    __syncthreads();
    for (int t = threadIdx.x; t < 16 * R; t += blockDim.x) {
      const int r_ = t / R, c_ = t - r_ * R;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < K1_WAVES; ++w) s += dpart[w][r_][c_];
      if (row0 + r_ < M) D[(row0 + r_) * R + c_] = s;
    }
  }
}

template <typename XT, int NCB>
static hipError_t launch_k1_t(const void* X, int64_t M, int64_t K, int64_t ldx,
                              const float* inv_smooth, const uint16_t* L1t, int R,
                              uint8_t* a_codes, uint16_t* a_scales, float* D, hipStream_t stream) {
  // groups in flight per wave, sized so the ring fits the register budget of
  // two resident workgroups
  constexpr int NB = (sizeof(XT) == 2 && NCB <= 2) ? 2 : 1;
  const dim3 block(64 * k1_waves<NCB>()), grid(static_cast<unsigned>((M + 15) / 16));
  hipLaunchKernelGGL((k1_quant_down_kernel<XT, NCB, NB>), grid, block, 0, stream,
                     static_cast<const XT*>(X), M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales,
                     D);
  return hipGetLastError();
}

template <typename XT>
static hipError_t launch_k1_dtype(const void* X, int64_t M, int64_t K, int64_t ldx,
                                  const float* inv_smooth, const uint16_t* L1t, int R,
                                  uint8_t* a_codes, uint16_t* a_scales, float* D,
                                  hipStream_t stream) {
  switch (R / 16) {
    case 0: return launch_k1_t<XT, 0>(X, M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales, D, stream);
    case 1: return launch_k1_t<XT, 1>(X, M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales, D, stream);
    case 2: return launch_k1_t<XT, 2>(X, M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales, D, stream);
    case 3: return launch_k1_t<XT, 3>(X, M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales, D, stream);
    case 4: return launch_k1_t<XT, 4>(X, M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales, D, stream);
    case 5: return launch_k1_t<XT, 5>(X, M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales, D, stream);
    case 6: return launch_k1_t<XT, 6>(X, M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales, D, stream);
    case 7:
    case 8: return launch_k1_t<XT, 8>(X, M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales, D, stream);
    default: return launch_k1_t<XT, 16>(X, M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales, D, stream);
  }
}

hipError_t launch_k1(const void* X, bool x_f16, int64_t M, int64_t K, int64_t ldx,
                     const float* inv_smooth, const uint16_t* L1t, int R, uint8_t* a_codes,
                     uint16_t* a_scales, float* D, hipStream_t stream) {
  if (x_f16)
    return launch_k1_dtype<_Float16>(X, M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales, D, stream);
  return launch_k1_dtype<float>(X, M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales, D, stream);
}

}  // namespace svdq
