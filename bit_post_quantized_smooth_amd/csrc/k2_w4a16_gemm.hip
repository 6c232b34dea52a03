// The 4-bit weight-only baseline (W4A16) of the SVDQuant abstract's speed
// comparison (ai-digest.ru page: 3.0x faster than a 4-bit weight-only
// baseline), built for gfx950 so that the comparison can be made on this GPU.
//
//   Y = fp16(X) . fp16(s q)^T + bias:
// 4-bit weights with one fp16 scale per 64 input channels, fp16 activations,
// the weights dequantized to fp16 on the fly and fed with the activations to
// v_mfma_f32_16x16x32_f16 (fp32 accumulation). No smoothing, no low-rank
// branch: the baseline quantizes only the weights.
//
// Layouts (svdq.h): the activation is first copied into a tiled fp16 layout
// by a small pass (tile_x_kernel), so that the GEMM's loads, like K2-MX's,
// are one contiguous 1 KB run per 16 rows and step of 32 along K; the weights
// are tiled offline, 256 bytes per 16 columns and step, with each code stored
// as code + 8.
//
// Dequantization of one lane's 8 codes (one 32-bit word u, nibble i = element
// i): (u >> 4p) & 0x000F000F | 0x64006400 is the fp16 pair (1024 + c_p + 8,
// 1024 + c_{p+4} + 8); subtracting 1032 is exact, multiplying by the scale
// rounds once: fp16(s c). The pairs come out in the element order 0, 4, 1, 5,
// 2, 6, 3, 7, and the activation tiles hold their 8 values in the same order,
// so the matrix instruction pairs every k with itself.
//
// Tiling as K2-MX: 256-thread workgroups of 2 x 2 waves, each wave a WTM x WTN
// block of the output (128 x 64: 8 activation blocks, whose fp16 operands are
// the heavier, share each dequantized weight fragment; measured faster than
// 64 x 128, 64 x 64 and 32 x 128), its operands loaded straight into registers
// with two steps in flight and a branch-free K loop; a thin last round in
// quarter tiles.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.hpp"
#include "device_launch.hpp"
#include "k2_common.hpp"

namespace svdq {

namespace {

constexpr int NT = 256;
constexpr int kStep = 32;            // K values per matrix instruction
constexpr int kXBlock = 512;         // fp16 per tiled activation block (16 rows x 32)
constexpr int kWBlock = 256;         // bytes per tiled weight block (16 columns x 32 codes)
constexpr int kSBlock = 64;          // fp16 scales per block (64 columns x one group)
constexpr int NS = 2;                // steps in flight per wave

template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// ---------------------------------------------------------------------------
// X -> x_t. A workgroup copies 16 rows x 128 channels (4 steps): thread t reads
// 16 contiguous bytes of X (8 channels; a row's 256 bytes come from 16
// consecutive threads) and writes them, reordered, to one lane slot.

template <typename XT>
__global__ __launch_bounds__(NT) void tile_x_kernel(const XT* __restrict__ X, int64_t M, int64_t K,
                                                    int64_t ldx, uint16_t* __restrict__ x_t) {
  const int t = threadIdx.x;
  const int64_t b = blockIdx.x;                     // 16-row block
  const int64_t S = K / kStep;
  const int row = t >> 4, piece = t & 15;           // piece: 8 channels
  const int64_t s = static_cast<int64_t>(blockIdx.y) * 4 + (piece >> 2);
  if (s >= S) return;                               // K % 128 == 64: the last copy has 2 steps
  const int q = piece & 3;
  int64_t m = b * 16 + row;
  m = m < M ? m : M - 1;
  const XT* src = X + m * ldx + s * kStep + 8 * q;
  float v[8];
  if constexpr (sizeof(XT) == 2) {
    const uint4 w = *reinterpret_cast<const uint4*>(src);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = h2f(static_cast<uint16_t>(ws[i] & 0xFFFFu));
      v[2 * i + 1] = h2f(static_cast<uint16_t>(ws[i] >> 16));
    }
  } else {
    const float4 a = reinterpret_cast<const float4*>(src)[0];
    const float4 c = reinterpret_cast<const float4*>(src)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
  }
  // element order 0, 4, 1, 5, 2, 6, 3, 7 (fp16 values round-trip exactly)
  const uint4 out = make_uint4(f2h(v[0]) | (static_cast<uint32_t>(f2h(v[4])) << 16),
                               f2h(v[1]) | (static_cast<uint32_t>(f2h(v[5])) << 16),
                               f2h(v[2]) | (static_cast<uint32_t>(f2h(v[6])) << 16),
                               f2h(v[3]) | (static_cast<uint32_t>(f2h(v[7])) << 16));
  *reinterpret_cast<uint4*>(x_t + ((b * S + s) * 64 + 16 * q + row) * 8) = out;
}

// ---------------------------------------------------------------------------
// GEMM

template <int NBM, int NBN>
struct W16Frags {
  static constexpr int SN = (NBN + 3) / 4;
  uint4 A[NBM];          // 8 fp16 activations per lane and row block
  uint32_t B[NBN];       // 8 offset-binary codes per lane and column block
  uint2 sc[SN];          // 4 fp16 scales (column blocks j = 0..3 of a 64-column group)
};

// fp16(s * c) for the 8 codes of u, in the element order 0, 4, 1, 5, 2, 6, 3, 7
__device__ __forceinline__ v8h dequant8(uint32_t u, _Float16 s) {
  const v2h off = v2h{static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
  const v2h sc = v2h{s, s};
  v2h h[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t bits = ((u >> (4 * p)) & 0x000F000Fu) | 0x64006400u;
    h[p] = (__builtin_bit_cast(v2h, bits) - off) * sc;     // exact, then one rounding
  }
  return v8h{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
}

template <int WTM, int WTN, bool Y_F16>
__device__ __forceinline__ void w16_tile(const uint16_t* __restrict__ x_t,
                                         const uint8_t* __restrict__ w_codes_t,
                                         const uint16_t* __restrict__ w_scales_t,
                                         const float* __restrict__ bias, void* __restrict__ Y,
                                         int64_t M, int64_t N, int64_t K, int64_t ldy, int64_t m0,
                                         int64_t n0, uint8_t* ystage) {
  constexpr int NBM = WTM / 16, NBN = WTN / 16;
  using Frags = W16Frags<NBM, NBN>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15;
  const int64_t S = K / kStep, G = K / kGroup;
  const int64_t ms = m0 + wm * WTM, ns = n0 + wn * WTN;
  const int64_t mb_last = (M + 15) / 16 - 1, nb_last = (N + 15) / 16 - 1;
  const int64_t ng_last = (N + 63) / 64 - 1;

  const uint16_t* ab[NBM];
  const uint8_t* bb[NBN];
  const uint16_t* sb[Frags::SN];
#pragma unroll
  for (int i = 0; i < NBM; ++i) {
    const int64_t b = ms / 16 + i;
    ab[i] = x_t + (b < mb_last ? b : mb_last) * S * kXBlock;
  }
#pragma unroll
  for (int j = 0; j < NBN; ++j) {
    const int64_t b = ns / 16 + j;
    bb[j] = w_codes_t + (b < nb_last ? b : nb_last) * S * kWBlock;
  }
#pragma unroll
  for (int c = 0; c < Frags::SN; ++c) {
    const int64_t g = ns / 64 + c;
    sb[c] = w_scales_t + (g < ng_last ? g : ng_last) * G * kSBlock;
  }
  // a wave of 32 columns that starts 32 columns into its 64-column group takes
  // the upper two of the four scales
  const int jsh = WTN < 64 ? static_cast<int>((ns % 64) / 16) : 0;

  auto load = [&](Frags& f, int64_t s) {
    s = s < S ? s : S - 1;
    const int64_t g = s >> 1;
#pragma unroll
    for (int i = 0; i < NBM; ++i)
      f.A[i] = *reinterpret_cast<const uint4*>(ab[i] + s * kXBlock + 8 * lane);
#pragma unroll
    for (int j = 0; j < NBN; ++j)
      f.B[j] = *reinterpret_cast<const uint32_t*>(bb[j] + s * kWBlock + 4 * lane);
#pragma unroll
    for (int c = 0; c < Frags::SN; ++c)
      f.sc[c] = *reinterpret_cast<const uint2*>(sb[c] + g * kSBlock + 4 * r);
  };

  v4f acc[NBM][NBN];
#pragma unroll
  for (int i = 0; i < NBM; ++i)
#pragma unroll
    for (int j = 0; j < NBN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto step = [&](const Frags& f) {
#pragma unroll
    for (int j = 0; j < NBN; ++j) {
      const int jj = (j % 4) + jsh;
      const uint2 w = f.sc[j / 4];
      const uint32_t half = jj < 2 ? w.x : w.y;
      const uint16_t sbits = static_cast<uint16_t>((jj & 1) ? (half >> 16) : (half & 0xFFFFu));
      const v8h bw = dequant8(f.B[j], __builtin_bit_cast(_Float16, sbits));
#pragma unroll
      for (int i = 0; i < NBM; ++i)
        acc[i][j] = mfma_f16_16x16x32(bw, __builtin_bit_cast(v8h, f.A[i]), acc[i][j]);
    }
  };

  Frags f[NS];
  static_for<NS>([&](auto P) { load(f[P.value], P.value); });
  int64_t s0 = 0;
  for (; s0 + NS <= S; s0 += NS) {
    static_for<NS>([&](auto P) {
      step(f[P.value]);
      __builtin_amdgcn_sched_barrier(0);
      load(f[P.value], s0 + P.value + NS);
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  static_for<NS>([&](auto P) {
    if (s0 + P.value < S) step(f[P.value]);
  });

  // full quarters of an fp16 Y go out through LDS in whole cache lines; the
  // staging area is used by nothing else, so no wave waits for another
  if constexpr (Y_F16 && WTN == 64) {
    if (ystage != nullptr && lds_store_ok<WTM, WTN>(Y, ldy, M, N, m0, n0)) {
      const int wave = threadIdx.x >> 6;
      bias_store_lds_f16<WTM, WTN, false>(acc, bias, static_cast<_Float16*>(Y), ldy, m0, n0,
                                          ystage + wave * WTM * 128);
      return;
    }
  }
  lowrank_bias_store<WTM, WTN, Y_F16, false>(acc, nullptr, nullptr, 0, bias, Y, M, N, ldy, m0,
                                             n0);
}

#ifndef W16_WTM
#define W16_WTM 128
#endif
#ifndef W16_WTN
#define W16_WTN 64
#endif
constexpr int kWtm = W16_WTM, kWtn = W16_WTN;       // wave tile of full workgroups
constexpr int kFullM = 2 * kWtm, kFullN = 2 * kWtn;  // full tile; quarters are half each way

template <bool Y_F16>
__global__ __launch_bounds__(NT, 2) void k2_w4a16_kernel(
    const uint16_t* __restrict__ x_t, const uint8_t* __restrict__ w_codes_t,
    const uint16_t* __restrict__ w_scales_t, const float* __restrict__ bias,
    void* __restrict__ Y, int64_t M, int64_t N, int64_t K, int64_t ldy, int tiles_m, int tiles_n,
    int n_full) {
  // Y staging of a full tile (fp16 only)
  __shared__ __attribute__((aligned(16))) uint8_t ystage[Y_F16 ? 4 * kWtm * 128 : 16];
  const int b = static_cast<int>(blockIdx.x);
  int tm, tn;
  if (b < n_full) {
    banded_tile(xcd_contiguous(b, n_full), tiles_m, tiles_n, tm, tn);
    w16_tile<kWtm, kWtn, Y_F16>(x_t, w_codes_t, w_scales_t, bias, Y, M, N, K, ldy,
                                static_cast<int64_t>(tm) * kFullM,
                                static_cast<int64_t>(tn) * kFullN, Y_F16 ? ystage : nullptr);
  } else {
    const int qb = b - n_full;
    const int quarter = qb & 3;
    banded_tile(n_full + (qb >> 2), tiles_m, tiles_n, tm, tn);
    w16_tile<kWtm / 2, kWtn / 2, Y_F16>(x_t, w_codes_t, w_scales_t, bias, Y, M, N, K, ldy,
                                        static_cast<int64_t>(tm) * kFullM + kWtm * (quarter >> 1),
                                        static_cast<int64_t>(tn) * kFullN + kWtn * (quarter & 1),
                                        nullptr);
  }
}

}  // namespace

hipError_t launch_w4a16_tile_x(const void* X, bool x_f16, int64_t M, int64_t K, int64_t ldx,
                               uint16_t* x_t, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((M + 15) / 16), static_cast<unsigned>((K / kStep + 3) / 4));
  if (x_f16)
    hipLaunchKernelGGL(tile_x_kernel<_Float16>, grid, dim3(NT), 0, stream,
                       static_cast<const _Float16*>(X), M, K, ldx, x_t);
  else
    hipLaunchKernelGGL(tile_x_kernel<float>, grid, dim3(NT), 0, stream,
                       static_cast<const float*>(X), M, K, ldx, x_t);
  return hipGetLastError();
}

hipError_t launch_w4a16_gemm(const uint16_t* x_t, const uint8_t* w_codes_t,
                             const uint16_t* w_scales_t, const float* bias, void* Y, bool y_f16,
                             int64_t M, int64_t N, int64_t K, int64_t ldy, hipStream_t stream) {
  const int tiles_m = static_cast<int>((M + kFullM - 1) / kFullM);
  const int tiles_n = static_cast<int>((N + kFullN - 1) / kFullN);
  const int T = tiles_m * tiles_n;
  // leftover tiles of the last round; quartered when they would fill at most
  // a quarter of the resident slots
  const int S = resident_slots();
  const int left = T < S ? T : T % S;
  const int n_quarter_tiles = (left > 0 && 4 * left <= S) ? left : 0;
  const int n_full = T - n_quarter_tiles;
  const dim3 grid(static_cast<unsigned>(n_full + 4 * n_quarter_tiles)), block(NT);
  if (y_f16)
    hipLaunchKernelGGL(k2_w4a16_kernel<true>, grid, block, 0, stream, x_t, w_codes_t, w_scales_t,
                       bias, Y, M, N, K, ldy, tiles_m, tiles_n, n_full);
  else
    hipLaunchKernelGGL(k2_w4a16_kernel<false>, grid, block, 0, stream, x_t, w_codes_t, w_scales_t,
                       bias, Y, M, N, K, ldy, tiles_m, tiles_n, n_full);
  return hipGetLastError();
}

}  // namespace svdq
