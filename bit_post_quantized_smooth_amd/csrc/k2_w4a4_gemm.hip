// K2: the W4A4 GEMM of the SVDQuant linear layer with the low-rank
// up-projection and the bias fused in (gfx950).
//
// Both operands are 4-bit (SVDQuant abstract: weights and activations at
// 4 bits; chattools.cn overview, section "SVDQuant的主要功能", quantization
// item). gfx950 has no 4-bit integer matrix instruction, so the nibbles are
// widened in registers to int8 lanes holding 16*q (two bit operations per 4
// codes, see device_common.hpp) and fed to v_mfma_i32_16x16x64_i8: one
// instruction covers exactly one 64-channel group of a 16x16 output block, so
// its int32 result is the exact group partial (times 256).
//
// Per-group rescale: the int32 accumulator is seeded with the bit pattern of
// 1.5*2^23, so the partial reads back as the float 12582912 + 256 P. Then
//     t   = fma(f, s_w / 256, -49152 * s_w)  = P * s_w  rounded once (fp32)
//     acc = fma(t, s_x, acc)
// i.e. two fp32 ops per output and group. The low-rank branch (the Nunchaku
// engine fuses it into the low-bit kernel: SVDQuant abstract; the
// disruptive-concepts.com post, section "Nunchaku: Fusing Precision and
// Speed") runs after the K loop as fp16 MFMAs on the same fp32 accumulators:
// acc += fp16(D) . L2, then the bias, then one rounding to the output type.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of Y; each of its
// 4 waves owns a 64 x 64 sub-tile (4 x 4 blocks of 16 x 16). The K loop moves
// 4 groups (128 bytes of codes per row) per stage through double-buffered LDS;
// each row's 32-byte group slice is stored as four 8-byte chunks XOR-swizzled
// by (row / 4) % 4, so the 16 lanes that read one chunk position from 16
// consecutive rows hit 16 different bank pairs.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "device_launch.hpp"

namespace svdq {

namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int KG = 4;               // groups per LDS stage
constexpr int NT = 256;             // threads per workgroup
static_assert(BM == BN && BM == 128 && NT == 2 * BM, "loader assumes 128 x 128 tiles");

struct StageRegs {
  uint4 a[4];                       // 64 bytes of A codes (2 groups of one row)
  uint4 b[4];                       // 64 bytes of B codes
  uint16_t sc[4];                   // scales of 4 groups: A row t (t < 128) or B row t-128
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

__device__ __forceinline__ void load_stage(StageRegs& r, const uint8_t* __restrict__ a_codes,
                                           const uint16_t* __restrict__ a_scales,
                                           const uint8_t* __restrict__ w_codes,
                                           const uint16_t* __restrict__ w_scales, int64_t M,
                                           int64_t N, int64_t K, int64_t G, int64_t m0, int64_t n0,
                                           int64_t g0) {
  const int t = threadIdx.x;
  const int row = t >> 1, half = t & 1;
  const int64_t kb = K / 2;
  const int64_t ga = g0 + 2 * half;                 // first group of this thread's 64 bytes
  // A codes
  {
    const int64_t m = m0 + row;
    const uint8_t* p = a_codes + m * kb + ga * kGroupBytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t g = ga + (j >> 1);
      r.a[j] = (m < M && g < G) ? *reinterpret_cast<const uint4*>(p + 16 * j) : make_uint4(0, 0, 0, 0);
    }
  }
  {
    const int64_t n = n0 + row;
    const uint8_t* p = w_codes + n * kb + ga * kGroupBytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t g = ga + (j >> 1);
      r.b[j] = (n < N && g < G) ? *reinterpret_cast<const uint4*>(p + 16 * j) : make_uint4(0, 0, 0, 0);
    }
  }
  {
    const bool is_a = t < BM;
    const int64_t idx = (is_a ? m0 : n0) + (t & (BM - 1));
    const bool ok = idx < (is_a ? M : N);
    const uint16_t* src = (is_a ? a_scales : w_scales) + idx * G;
#pragma unroll
    for (int j = 0; j < KG; ++j) r.sc[j] = (ok && g0 + j < G) ? src[g0 + j] : 0;
  }
}

struct Smem {
  uint8_t a[2][KG][BM][kGroupBytes];
  uint8_t b[2][KG][BN][kGroupBytes];
  uint16_t sc[2][KG][2][BM];        // [.][.][0][row] = A scales, [.][.][1][col] = B scales
};

__device__ __forceinline__ void store_stage(const StageRegs& r, Smem& sm, int buf) {
  const int t = threadIdx.x;
  const int row = t >> 1, half = t & 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int gg = 2 * half + (j >> 1);
    const int c0 = 2 * (j & 1);                     // chunk index of the first 8 bytes
    uint2 lo = make_uint2(r.a[j].x, r.a[j].y), hi = make_uint2(r.a[j].z, r.a[j].w);
    *reinterpret_cast<uint2*>(&sm.a[buf][gg][row][8 * swz(row, c0)]) = lo;
    *reinterpret_cast<uint2*>(&sm.a[buf][gg][row][8 * swz(row, c0 + 1)]) = hi;
    lo = make_uint2(r.b[j].x, r.b[j].y);
    hi = make_uint2(r.b[j].z, r.b[j].w);
    *reinterpret_cast<uint2*>(&sm.b[buf][gg][row][8 * swz(row, c0)]) = lo;
    *reinterpret_cast<uint2*>(&sm.b[buf][gg][row][8 * swz(row, c0 + 1)]) = hi;
  }
#pragma unroll
  for (int j = 0; j < KG; ++j) sm.sc[buf][j][t >> 7][t & (BM - 1)] = r.sc[j];
}

template <bool Y_F16>
__global__ __launch_bounds__(NT) void k2_w4a4_kernel(
    const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
    const uint8_t* __restrict__ w_codes, const uint16_t* __restrict__ w_scales,
    const float* __restrict__ D, const uint16_t* __restrict__ L2t, int R,
    const float* __restrict__ bias, void* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int tiles_n) {
  __shared__ Smem sm;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int tile = blockIdx.x;
  const int64_t m0 = static_cast<int64_t>(tile / tiles_n) * BM;
  const int64_t n0 = static_cast<int64_t>(tile % tiles_n) * BN;
  const int64_t G = K / kGroup;
  const int64_t S = (G + KG - 1) / KG;

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4i seed = v4i{kMagicSeed, kMagicSeed, kMagicSeed, kMagicSeed};

  StageRegs st;
  load_stage(st, a_codes, a_scales, w_codes, w_scales, M, N, K, G, m0, n0, 0);
  store_stage(st, sm, 0);
  __syncthreads();

  for (int64_t s = 0; s < S; ++s) {
    const int buf = static_cast<int>(s & 1);
    if (s + 1 < S)
      load_stage(st, a_codes, a_scales, w_codes, w_scales, M, N, K, G, m0, n0, (s + 1) * KG);
#pragma unroll 1
    for (int gg = 0; gg < KG; ++gg) {
      v4i A[4], B[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + rl;
        A[i] = widen_codes(*reinterpret_cast<const uint2*>(&sm.a[buf][gg][r][8 * swz(r, q)]));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = wn * 64 + j * 16 + rl;
        B[j] = widen_codes(*reinterpret_cast<const uint2*>(&sm.b[buf][gg][c][8 * swz(c, q)]));
      }
      float sx[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint2 p = *reinterpret_cast<const uint2*>(&sm.sc[buf][gg][0][wm * 64 + i * 16 + 4 * q]);
        sx[i][0] = h2f(static_cast<uint16_t>(p.x & 0xFFFFu));
        sx[i][1] = h2f(static_cast<uint16_t>(p.x >> 16));
        sx[i][2] = h2f(static_cast<uint16_t>(p.y & 0xFFFFu));
        sx[i][3] = h2f(static_cast<uint16_t>(p.y >> 16));
      }
      float al[4], be[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sw = h2f(sm.sc[buf][gg][1][wn * 64 + j * 16 + rl]);
        al[j] = sw * 0.00390625f;                 // s_w / 256, exact
        be[j] = sw * -49152.0f;                   // -(1.5 * 2^23 / 256) s_w, exact
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4i p = mfma_i8_16x16x64(A[i], B[j], seed);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int pe = p[e];                 // scalar copy: see as_float()
            const float f = as_float(pe);
            const float t = __builtin_fmaf(f, al[j], be[j]);
            acc[i][j][e] = __builtin_fmaf(t, sx[i][e], acc[i][j][e]);
          }
        }
      }
    }
    if (s + 1 < S) store_stage(st, sm, buf ^ 1);
    __syncthreads();
  }

  // low-rank up-projection on the same accumulators: acc += fp16(D) . L2
  for (int rc = 0; rc < R; rc += 32) {
    const int kk = rc + 8 * q;                       // this lane's 8 rank indices
    const bool kval = kk < R;                        // R % 16 == 0: whole 8-runs are valid or not
    v8h Al[4], Bl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wm * 64 + i * 16 + rl;
      if (kval && m < M) {
        const float4* dp = reinterpret_cast<const float4*>(D + m * R + kk);
        const float4 u = dp[0], v = dp[1];
        Al[i] = v8h{static_cast<_Float16>(u.x), static_cast<_Float16>(u.y),
                    static_cast<_Float16>(u.z), static_cast<_Float16>(u.w),
                    static_cast<_Float16>(v.x), static_cast<_Float16>(v.y),
                    static_cast<_Float16>(v.z), static_cast<_Float16>(v.w)};
      } else {
        Al[i] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 64 + j * 16 + rl;
      if (kval && n < N)
        Bl[j] = *reinterpret_cast<const v8h*>(L2t + n * R + kk);
      else
        Bl[j] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f16_16x16x32(Al[i], Bl[j], acc[i][j]);
  }

  // bias and store; lane holds rows 4q+e of column rl in each 16 x 16 block
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t n = n0 + wn * 64 + j * 16 + rl;
    if (n >= N) continue;
    const float b = bias ? bias[n] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + wm * 64 + i * 16 + 4 * q + e;
        if (m < M) {
          const float v = acc[i][j][e] + b;
          if constexpr (Y_F16)
            static_cast<_Float16*>(Y)[m * ldy + n] = static_cast<_Float16>(v);
          else
            static_cast<float*>(Y)[m * ldy + n] = v;
        }
      }
    }
  }
}

// Exact integer partials for a slice of rows, with the same operand widening
// and the same int8 matrix instruction as the GEMM. One wave per 16 x 16 block.
__global__ __launch_bounds__(64) void debug_partials_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ w_codes, int64_t M, int64_t N,
    int64_t K, int64_t row0, int64_t rows, int32_t* __restrict__ P) {
  const int lane = threadIdx.x;
  const int rl = lane & 15, q = lane >> 4;
  const int64_t rb = static_cast<int64_t>(blockIdx.x) * 16;     // offset inside the slice
  const int64_t cb = static_cast<int64_t>(blockIdx.y) * 16;
  const int64_t G = K / kGroup, kb = K / 2;
  const int64_t ra = row0 + rb + rl;                              // row this lane loads
  const int64_t nb = cb + rl;                                     // column this lane loads
  for (int64_t g = 0; g < G; ++g) {
    uint2 pa = make_uint2(0, 0), pb = make_uint2(0, 0);
    if (rb + rl < rows && ra < M)
      pa = *reinterpret_cast<const uint2*>(a_codes + ra * kb + g * kGroupBytes + 8 * q);
    if (nb < N) pb = *reinterpret_cast<const uint2*>(w_codes + nb * kb + g * kGroupBytes + 8 * q);
    const v4i r = mfma_i8_16x16x64(widen_codes(pa), widen_codes(pb), v4i{0, 0, 0, 0});
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t mr = rb + 4 * q + e;                          // output row inside the slice
      if (mr < rows && nb < N) P[(mr * N + nb) * G + g] = r[e] >> 8;   // 256 P -> P, exact
    }
  }
}

}  // namespace

hipError_t launch_k2(const uint8_t* a_codes, const uint16_t* a_scales, const uint8_t* w_codes,
                     const uint16_t* w_scales, const float* D, const uint16_t* L2t, int R,
                     const float* bias, void* Y, bool y_f16, int64_t M, int64_t N, int64_t K,
                     int64_t ldy, hipStream_t stream) {
  const int tiles_m = static_cast<int>((M + BM - 1) / BM);
  const int tiles_n = static_cast<int>((N + BN - 1) / BN);
  const dim3 grid(static_cast<unsigned>(tiles_m) * tiles_n), block(NT);
  if (y_f16)
    hipLaunchKernelGGL(k2_w4a4_kernel<true>, grid, block, 0, stream, a_codes, a_scales, w_codes,
                       w_scales, D, L2t, R, bias, Y, M, N, K, ldy, tiles_n);
  else
    hipLaunchKernelGGL(k2_w4a4_kernel<false>, grid, block, 0, stream, a_codes, a_scales, w_codes,
                       w_scales, D, L2t, R, bias, Y, M, N, K, ldy, tiles_n);
  return hipGetLastError();
}

hipError_t launch_debug_partials(const uint8_t* a_codes, const uint8_t* w_codes, int64_t M,
                                 int64_t N, int64_t K, int64_t row0, int64_t rows, int32_t* P,
                                 hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((rows + 15) / 16), static_cast<unsigned>((N + 15) / 16));
  hipLaunchKernelGGL(debug_partials_kernel, grid, dim3(64), 0, stream, a_codes, w_codes, M, N, K,
                     row0, rows, P);
  return hipGetLastError();
}

}  // namespace svdq
