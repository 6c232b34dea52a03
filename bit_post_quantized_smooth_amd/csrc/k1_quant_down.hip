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
// Work split: a workgroup owns 16 rows; its waves take the 64-channel groups
// round-robin, so consecutive groups of a row are in flight in neighbouring
// waves and each wave's loads are 16 rows x 128 contiguous bytes. Lane l
// handles row l%16 and the 16 channels 16*(l/16) .. +15 of the group: these
// 16 values are both its quantizer input and, rounded to fp16, its operand
// pieces for v_mfma_f32_16x16x32_f16 (the matching L1 values come from the
// same channels, so the two operands agree on the summation order). The
// per-wave partial D tiles are summed in LDS in a fixed order.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "device_launch.hpp"

namespace svdq {

template <typename XT>
__device__ __forceinline__ void load16(const XT* p, float* v);

template <>
__device__ __forceinline__ void load16<_Float16>(const _Float16* p, float* v) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 a = q[0], b = q[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = h2f(static_cast<uint16_t>(w[i] & 0xFFFFu));
    v[2 * i + 1] = h2f(static_cast<uint16_t>(w[i] >> 16));
  }
}

template <>
__device__ __forceinline__ void load16<float>(const float* p, float* v) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float4 t = q[i];
    v[4 * i] = t.x;
    v[4 * i + 1] = t.y;
    v[4 * i + 2] = t.z;
    v[4 * i + 3] = t.w;
  }
}

// NCB = number of 16-wide column blocks of D handled with registers sized at
// compile time; `ncb` <= NCB is the runtime count (R / 16).
template <typename XT, int NCB>
__global__ __launch_bounds__(512) void k1_quant_down_kernel(
    const XT* __restrict__ X, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ inv_smooth, const uint16_t* __restrict__ L1t, int R,
    uint8_t* __restrict__ a_codes, uint16_t* __restrict__ a_scales, float* __restrict__ D) {
#pragma clang fp contract(off)
  extern __shared__ float dpart[];   // [waves][16][R]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int rl = lane & 15, q = lane >> 4;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t row = row0 + rl;
  const bool rvalid = row < M;
  const int64_t G = K / kGroup;
  const int ncb = R / 16;

  v4f acc[NCB > 0 ? NCB : 1];
#pragma unroll
  for (int c = 0; c < (NCB > 0 ? NCB : 1); ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int64_t g = wave; g < G; g += nwaves) {
    const int64_t k0 = g * kGroup + q * 16;
    float xv[16];
    if (rvalid) {
      load16<XT>(X + row * ldx + k0, xv);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) xv[i] = 0.f;
    }
    const float4* ip = reinterpret_cast<const float4*>(inv_smooth + k0);
    float xh[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 s = ip[i];
      xh[4 * i + 0] = xv[4 * i + 0] * s.x;
      xh[4 * i + 1] = xv[4 * i + 1] * s.y;
      xh[4 * i + 2] = xv[4 * i + 2] * s.z;
      xh[4 * i + 3] = xv[4 * i + 3] * s.w;
    }
    // group absmax over this lane's 16 values, then across the 4 lanes of the row
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(xh[i]));
    a = fmaxf(a, __shfl_xor(a, 16));
    a = fmaxf(a, __shfl_xor(a, 32));
    const float s32 = fminf(a / 7.0f, 65504.0f);      // correctly rounded division
    const uint16_t s16 = f2h(s32);
    const float sf = h2f(s16);
    const float inv = (sf == 0.f) ? 0.f : 1.0f / sf;
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float t = rintf(xh[i] * inv);                    // half-to-even
      t = fminf(fmaxf(t, -7.f), 7.f);
      const uint32_t nib = static_cast<uint32_t>(static_cast<int>(t)) & 0xFu;
      packed[i >> 3] |= nib << (4 * (i & 7));
    }
    if (rvalid) {
      *reinterpret_cast<uint2*>(a_codes + row * (K / 2) + g * kGroupBytes + q * 8) =
          make_uint2(packed[0], packed[1]);
      if (q == 0) a_scales[row * G + g] = s16;
    }
    if constexpr (NCB > 0) {
      v8h x0, x1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x0[i] = static_cast<_Float16>(xh[i]);
        x1[i] = static_cast<_Float16>(xh[8 + i]);
      }
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        if (c < ncb) {
          const uint16_t* lp = L1t + static_cast<int64_t>(c * 16 + rl) * K + k0;
          const v8h b0 = *reinterpret_cast<const v8h*>(lp);
          const v8h b1 = *reinterpret_cast<const v8h*>(lp + 8);
          acc[c] = mfma_f16_16x16x32(x0, b0, acc[c]);
          acc[c] = mfma_f16_16x16x32(x1, b1, acc[c]);
        }
      }
    }
  }

  if constexpr (NCB > 0) {
    // partial D of this wave -> LDS; lane holds rows 4q+i of column c*16+rl
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      if (c < ncb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dpart[(wave * 16 + 4 * q + i) * R + c * 16 + rl] = acc[c][i];
      }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < 16 * R; t += blockDim.x) {
      const int r_ = t / R, c_ = t - r_ * R;
      float s = 0.f;
      for (int w = 0; w < nwaves; ++w) s += dpart[(w * 16 + r_) * R + c_];
      if (row0 + r_ < M) D[(row0 + r_) * R + c_] = s;
    }
  }
}

template <typename XT, int NCB>
static hipError_t launch_k1_t(const void* X, int64_t M, int64_t K, int64_t ldx,
                              const float* inv_smooth, const uint16_t* L1t, int R,
                              uint8_t* a_codes, uint16_t* a_scales, float* D, hipStream_t stream) {
  const int64_t G = K / kGroup;
  int waves = static_cast<int>(G < 8 ? G : 8);
  // keep the D-reduction buffer within 64 KiB of LDS
  while (NCB > 0 && waves > 1 && sizeof(float) * waves * 16 * R > 65536) --waves;
  const dim3 block(64 * waves), grid(static_cast<unsigned>((M + 15) / 16));
  const size_t lds = NCB > 0 ? sizeof(float) * waves * 16 * R : 0;
  hipLaunchKernelGGL((k1_quant_down_kernel<XT, NCB>), grid, block, lds, stream,
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
    case 3:
    case 4: return launch_k1_t<XT, 4>(X, M, K, ldx, inv_smooth, L1t, R, a_codes, a_scales, D, stream);
    case 5:
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
