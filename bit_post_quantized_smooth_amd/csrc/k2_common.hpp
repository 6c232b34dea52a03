// Pieces shared by the GEMM kernels (INT4, MXFP4 and the weight-only
// baseline): the XCD-aware tile order (which the pre-kernel uses too) and the
// epilogue that adds the low-rank up-projection and the bias, applies the
// optional GELU and stores Y.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace svdq {

// Resident workgroup slots of the current device (2 per compute unit).
int resident_slots();

namespace {

// Tile order. Workgroups are dealt to the 8 XCDs round-robin (workgroup b runs
// on XCD b % 8), and each XCD has its own L2. Renumber so that every XCD works
// through one contiguous run of tiles, and walk the tiles in bands of
// kBandM tile rows, column by column: the tiles an XCD holds at one time then
// share a few A row panels and B column panels, which stay in its L2.
constexpr int kXcds = 8;
constexpr int kBandM = 4;   // measured against 2, 8, 16 and 36: 1-2% ahead of 8

__device__ __forceinline__ int xcd_contiguous(int b, int T) {
  const int per = T / kXcds, rem = T % kXcds;
  const int x = b % kXcds, local = b / kXcds;
  return x * per + (x < rem ? x : rem) + local;             // a bijection of [0, T)
}

__device__ __forceinline__ void banded_tile(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int band_tiles = kBandM * tiles_n;
  const int band = t / band_tiles;
  const int first_m = band * kBandM;
  const int rows = tiles_m - first_m < kBandM ? tiles_m - first_m : kBandM;
  const int r = t - band * band_tiles;
  tm = first_m + r % rows;
  tn = r / rows;
}

// Epilogue pieces of a 2*WTM x 2*WTN tile whose 4 waves each hold a WTM x WTN
// quarter in fp32 accumulators (wave w: rows wm = w/2, columns wn = w%2; in
// each 16 x 16 block a lane holds columns 4*(lane/16) .. +3 of row lane%16).
// The low-rank branch (the Nunchaku engine fuses it into the low-bit kernel:
// SVDQuant abstract; the disruptive-concepts.com post, section "Nunchaku:
// Fusing Precision and Speed") runs as fp16 MFMAs on the same accumulators:
// acc += fp16(D) . L2; then the bias, optionally the GELU, and one rounding
// to the output type.
// The low-rank up-projection on the accumulators: acc += fp16(D) . L2.
// Every load is unconditional, from a clamped in-bounds address, and
// out-of-range operands are zeroed after it arrives; a load under a branch
// whose other side zeroes the same registers would have to complete before
// anything else is issued.
// lowrank_up_at: for a wave whose WTM x WTN region of Y starts at row mw and
// column nw; lowrank_up: for the wave's quarter of a 2*WTM x 2*WTN tile at
// (m0, n0) (wave w: rows w/2, columns w%2).
template <int WTM, int WTN>
__device__ __forceinline__ void lowrank_up_at(v4f (&acc)[WTM / 16][WTN / 16],
                                              const float* __restrict__ D,
                                              const uint16_t* __restrict__ L2t, int R, int64_t M,
                                              int64_t N, int64_t mw, int64_t nw) {
  constexpr int NBM = WTM / 16, NBN = WTN / 16;
  const int lane = threadIdx.x & 63;
  const int rl = lane & 15, q = lane >> 4;
  const int64_t m0 = mw, n0 = nw;
  constexpr int wm = 0, wn = 0;
  const v8h zero = v8h{0, 0, 0, 0, 0, 0, 0, 0};
  for (int rc = 0; rc < R; rc += 32) {
    const int kk = rc + 8 * q;                       // this lane's 8 rank indices
    const bool kval = kk < R;                        // R % 16 == 0: whole 8-runs are valid or not
    v8h Bl[NBN];
#pragma unroll
    for (int j = 0; j < NBN; ++j) {
      const int64_t n = n0 + wn * WTN + j * 16 + rl;
      const bool ok = kval && n < N;
      const v8h b = *reinterpret_cast<const v8h*>(L2t + (ok ? n * R + kk : 0));
      Bl[j] = ok ? b : zero;
    }
#pragma unroll
    for (int i = 0; i < NBM; ++i) {
      const int64_t m = m0 + wm * WTM + i * 16 + rl;
      const bool ok = kval && m < M;
      const float4* dp = reinterpret_cast<const float4*>(D + (ok ? m * R + kk : 0));
      const float4 u = dp[0], v = dp[1];
      const v8h a = v8h{static_cast<_Float16>(u.x), static_cast<_Float16>(u.y),
                        static_cast<_Float16>(u.z), static_cast<_Float16>(u.w),
                        static_cast<_Float16>(v.x), static_cast<_Float16>(v.y),
                        static_cast<_Float16>(v.z), static_cast<_Float16>(v.w)};
      const v8h Al = ok ? a : zero;
#pragma unroll
      for (int j = 0; j < NBN; ++j) acc[i][j] = mfma_f16_16x16x32(Bl[j], Al, acc[i][j]);
    }
  }
}

template <int WTM, int WTN>
__device__ __forceinline__ void lowrank_up(v4f (&acc)[WTM / 16][WTN / 16],
                                           const float* __restrict__ D,
                                           const uint16_t* __restrict__ L2t, int R, int64_t M,
                                           int64_t N, int64_t m0, int64_t n0) {
  const int wave = threadIdx.x >> 6;
  lowrank_up_at<WTM, WTN>(acc, D, L2t, R, M, N, m0 + (wave >> 1) * WTM,
                          n0 + (wave & 1) * WTN);
}

// The same up-projection from the pre-kernel's fp16 D in operand order (D_t:
// per 16-row block and 32-rank chunk one 1 KB block, lane 16q + r holding row
// r, ranks 8q .. 8q+7; svdq.h, tiled layouts): one 16-byte load per row block
// and chunk, nothing converted. The same sums as lowrank_up_at, whose operand
// is the same fp16(D).
template <int WTM, int WTN>
__device__ __forceinline__ void lowrank_up_dt_at(v4f (&acc)[WTM / 16][WTN / 16],
                                                 const uint16_t* __restrict__ Dt,
                                                 const uint16_t* __restrict__ L2t, int R,
                                                 int64_t M, int64_t N, int64_t mw, int64_t nw) {
  constexpr int NBM = WTM / 16, NBN = WTN / 16;
  const int lane = threadIdx.x & 63;
  const int rl = lane & 15, q = lane >> 4;
  const int RC = (R + 31) / 32;
  const int64_t Mb = (M + 15) / 16;
  const v8h zero = v8h{0, 0, 0, 0, 0, 0, 0, 0};
  for (int c = 0; c < RC; ++c) {
    const int kk = 32 * c + 8 * q;                   // this lane's 8 rank indices
    const bool kval = kk < R;                        // R % 16 == 0: whole 8-runs are valid or not
    v8h Bl[NBN], Ar[NBM];
#pragma unroll
    for (int j = 0; j < NBN; ++j) {
      const int64_t n = nw + j * 16 + rl;
      const bool ok = kval && n < N;
      Bl[j] = *reinterpret_cast<const v8h*>(L2t + (ok ? n * R + kk : 0));
    }
#pragma unroll
    for (int i = 0; i < NBM; ++i) {
      int64_t b = mw / 16 + i;
      b = b < Mb ? b : Mb - 1;
      Ar[i] = *reinterpret_cast<const v8h*>(Dt + ((b * RC + c) * 64 + lane) * 8);
    }
#pragma unroll
    for (int j = 0; j < NBN; ++j) Bl[j] = (kval && nw + j * 16 + rl < N) ? Bl[j] : zero;
#pragma unroll
    for (int i = 0; i < NBM; ++i) {
      const v8h Al = (kval && mw + i * 16 + rl < M) ? Ar[i] : zero;
#pragma unroll
      for (int j = 0; j < NBN; ++j) acc[i][j] = mfma_f16_16x16x32(Bl[j], Al, acc[i][j]);
    }
  }
}

template <int WTM, int WTN>
__device__ __forceinline__ void lowrank_up_dt(v4f (&acc)[WTM / 16][WTN / 16],
                                              const uint16_t* __restrict__ Dt,
                                              const uint16_t* __restrict__ L2t, int R, int64_t M,
                                              int64_t N, int64_t m0, int64_t n0) {
  const int wave = threadIdx.x >> 6;
  lowrank_up_dt_at<WTM, WTN>(acc, Dt, L2t, R, M, N, m0 + (wave >> 1) * WTM,
                             n0 + (wave & 1) * WTN);
}

// Bias, the optional GELU, one rounding to the output type, and the stores: a
// lane holds columns 4q .. 4q+3 of row rl in each 16 x 16 block, written as
// one 8-byte (fp16) or 16-byte (fp32) store when Y's address and row stride
// allow it. bias_store_at: the wave's region starts at (mw, nw); bias_store:
// the wave's quarter of the tile at (m0, n0), as lowrank_up.
template <int WTM, int WTN, bool Y_F16, bool GELU>
__device__ __forceinline__ void bias_store_at(v4f (&acc)[WTM / 16][WTN / 16],
                                              const float* __restrict__ bias,
                                              void* __restrict__ Y, int64_t M, int64_t N,
                                              int64_t ldy, int64_t mw, int64_t nw) {
  constexpr int NBM = WTM / 16, NBN = WTN / 16;
  const int lane = threadIdx.x & 63;
  const int rl = lane & 15, q = lane >> 4;
  const int64_t m0 = mw, n0 = nw;
  constexpr int wm = 0, wn = 0;
  constexpr int ES = Y_F16 ? 2 : 4;
  const bool vec = ((reinterpret_cast<uintptr_t>(Y) | static_cast<uintptr_t>(ldy * ES)) %
                    (4 * ES)) == 0;
  float bv[NBN][4];
#pragma unroll
  for (int j = 0; j < NBN; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t n = n0 + wn * WTN + j * 16 + 4 * q + e;
      bv[j][e] = (bias != nullptr && n < N) ? bias[n] : 0.f;
    }
#pragma unroll
  for (int i = 0; i < NBM; ++i) {
    const int64_t m = m0 + wm * WTM + i * 16 + rl;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < NBN; ++j) {
      const int64_t n = n0 + wn * WTN + j * 16 + 4 * q;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = acc[i][j][e] + bv[j][e];
        if constexpr (GELU) v[e] = gelu_tanh_f32(v[e]);
      }
      if (vec && n + 3 < N) {
        if constexpr (Y_F16) {
          const uint32_t lo = static_cast<uint32_t>(f2h(v[0])) | (static_cast<uint32_t>(f2h(v[1])) << 16);
          const uint32_t hi = static_cast<uint32_t>(f2h(v[2])) | (static_cast<uint32_t>(f2h(v[3])) << 16);
          *reinterpret_cast<uint2*>(static_cast<_Float16*>(Y) + m * ldy + n) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(Y) + m * ldy + n) =
              make_float4(v[0], v[1], v[2], v[3]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (n + e < N) {
            if constexpr (Y_F16)
              static_cast<_Float16*>(Y)[m * ldy + n + e] = static_cast<_Float16>(v[e]);
            else
              static_cast<float*>(Y)[m * ldy + n + e] = v[e];
          }
        }
      }
    }
  }
}

template <int WTM, int WTN, bool Y_F16, bool GELU>
__device__ __forceinline__ void bias_store(v4f (&acc)[WTM / 16][WTN / 16],
                                           const float* __restrict__ bias, void* __restrict__ Y,
                                           int64_t M, int64_t N, int64_t ldy, int64_t m0,
                                           int64_t n0) {
  const int wave = threadIdx.x >> 6;
  bias_store_at<WTM, WTN, Y_F16, GELU>(acc, bias, Y, M, N, ldy, m0 + (wave >> 1) * WTM,
                                       n0 + (wave & 1) * WTN);
}

// The same epilogue for an fp16 Y through LDS, for a wave whose WTM x 64
// quarter lies inside Y, with Y and its row stride 16-byte aligned. The wave
// writes its rounded values (bias and GELU applied) into its own region of
// LDS (WTM rows of 128 bytes, the 16-byte units of row r XOR-swizzled by
// r % 8), then reads them back 16 bytes per lane: 8 lanes cover one 128-byte
// row, so every store instruction writes 8 whole cache lines of Y instead of
// 32-byte pieces of 16. `lds` is this wave's region (WTM * 128 bytes, 16-byte
// aligned); the caller makes sure no other wave still reads it.
template <int WTM, int WTN, bool GELU>
__device__ __forceinline__ void bias_store_lds_f16(v4f (&acc)[WTM / 16][WTN / 16],
                                                   const float* __restrict__ bias,
                                                   _Float16* __restrict__ Y, int64_t ldy,
                                                   int64_t m0, int64_t n0, uint8_t* lds) {
  static_assert(WTN == 64, "one 128-byte LDS row per output row");
  constexpr int NBM = WTM / 16, NBN = WTN / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rl = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t mw = m0 + wm * WTM, nw = n0 + wn * WTN;
  float bv[NBN][4];
#pragma unroll
  for (int j = 0; j < NBN; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) bv[j][e] = bias != nullptr ? bias[nw + j * 16 + 4 * q + e] : 0.f;
#pragma unroll
  for (int i = 0; i < NBM; ++i) {
    const int row = i * 16 + rl;
#pragma unroll
    for (int j = 0; j < NBN; ++j) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = acc[i][j][e] + bv[j][e];
        if constexpr (GELU) v[e] = gelu_tanh_f32(v[e]);
      }
      const uint32_t lo = static_cast<uint32_t>(f2h(v[0])) | (static_cast<uint32_t>(f2h(v[1])) << 16);
      const uint32_t hi = static_cast<uint32_t>(f2h(v[2])) | (static_cast<uint32_t>(f2h(v[3])) << 16);
      const int unit = 2 * j + (q >> 1);              // 16-byte unit of columns 16j + 4q .. +3
      *reinterpret_cast<uint2*>(lds + row * 128 + ((unit ^ (row & 7)) << 4) + ((q & 1) << 3)) =
          make_uint2(lo, hi);
    }
  }
  const int u = lane & 7, r8 = lane >> 3;
#pragma unroll
  for (int it = 0; it < WTM / 8; ++it) {
    const int row = it * 8 + r8;
    const uint4 v = *reinterpret_cast<const uint4*>(lds + row * 128 + ((u ^ r8) << 4));
    *reinterpret_cast<uint4*>(Y + (mw + row) * ldy + nw + 8 * u) = v;
  }
}

// Whether this wave's WTM x WTN quarter of the tile at (m0, n0) may take the
// LDS-staged fp16 store: inside Y, Y and its row stride 16-byte aligned.
template <int WTM, int WTN>
__device__ __forceinline__ bool lds_store_ok(const void* Y, int64_t ldy, int64_t M, int64_t N,
                                             int64_t m0, int64_t n0) {
  const int wave = threadIdx.x >> 6;
  const int64_t mw = m0 + (wave >> 1) * WTM, nw = n0 + (wave & 1) * WTN;
  return mw + WTM <= M && nw + WTN <= N &&
         ((reinterpret_cast<uintptr_t>(Y) | static_cast<uintptr_t>(ldy * 2)) % 16) == 0;
}

// Both, in that order (the INT4 and weight-only kernels' epilogue).
template <int WTM, int WTN, bool Y_F16, bool GELU>
__device__ __forceinline__ void lowrank_bias_store(
    v4f (&acc)[WTM / 16][WTN / 16], const float* __restrict__ D, const uint16_t* __restrict__ L2t,
    int R, const float* __restrict__ bias, void* __restrict__ Y, int64_t M, int64_t N,
    int64_t ldy, int64_t m0, int64_t n0) {
  lowrank_up<WTM, WTN>(acc, D, L2t, R, M, N, m0, n0);
  bias_store<WTM, WTN, Y_F16, GELU>(acc, bias, Y, M, N, ldy, m0, n0);
}

}  // namespace

}  // namespace svdq
