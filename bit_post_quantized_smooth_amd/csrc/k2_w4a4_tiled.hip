// K2T: the W4A4 GEMM of the SVDQuant linear layer on tiled operands, with the
// low-rank up-projection and the bias fused in (gfx950).
//
// The arithmetic is K2's (k2_w4a4_gemm.hip): both operands are 4-bit codes
// (SVDQuant abstract: weights and activations at 4 bits), widened to int8
// lanes holding 16*q for v_mfma_i32_16x16x64_i8, whose int32 result over one
// 64-channel group is the exact group partial P (times 256, read through the
// 1.5*2^23 accumulator seed as the float f = 12582912 + 256 P); per output
// and group two fp32 ops
//     t   = fma(f, s_w/256, -12582912 s_w/256) = P s_w   (exact)
//     acc = fma(t, s_x, acc)                            (the one rounding)
// and the low-rank branch fp16(D) . L2 and the bias in the same kernel (the
// Nunchaku engine fuses the low-rank kernels into the low-bit ones:
// SVDQuant abstract; the disruptive-concepts.com post, section "Nunchaku:
// Fusing Precision and Speed").
//
// Those two fp32 ops per output and group bound the kernel. Measured on this
// chip, a wave64 v_fma_f32 occupies a SIMD for about 2.5 cycles once two or
// more waves share it (one wave alone issues one every ~5 cycles), an i8
// 16x16x64 matrix instruction for about 17, and the two do not overlap: a
// SIMD running both spends the sum. Per group and wave that is 16 matrix
// instructions (272 cycles) against 128 rescale FMAs (~320 cycles), so the
// kernel keeps every other vector op out of the K loop:
// - the activation operand arrives already widened, in the matrix
//   instruction's lane order, from the pre-kernel (svdq.h, tiled INT4
//   layouts), with its scale in fp32;
// - the weights stay 4-bit (the 4-bit weight memory is the method's point)
//   in a lane-order tiling per 32-column strip, so a wave's weight fragment
//   for one group is one 16-byte read per lane, widened once (12 bit ops);
//   their scales arrive as the exact fp32 pairs (s_w/256, -12582912 s_w/256),
//   made once offline, so no scale is converted in the loop (an fp16 scale
//   folded into the FMAs as v_fma_mix_f32 would cost ~4.4 cycles an op
//   against ~2.5 for v_fma_f32);
// - every operand goes from global memory straight into LDS
//   (global_load_lds: no register round trip), KSTAGES groups deep, with one
//   barrier per group; addresses advance by scalar offsets.
// What remains per group and wave: 16 matrix instructions, 128 rescale ops,
// 12 widening ops, 9 address and other ops, 15 LDS reads and 5 copies. Three
// workgroups share a compute unit (142 registers, 41.5 KB of LDS), so a wave
// waiting at the barrier or on LDS leaves the SIMD to two others.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of Y; wave w owns
// all 128 rows and columns 32w .. 32w+31 (8 x 2 blocks of 16 x 16), so its
// weight strip is its own and only the activation operands are shared. The
// weight fragment is the matrix instruction's first operand, so a lane holds 4
// consecutive columns of one row of each block (as in K2). Tiles run in K2's
// XCD-aware banded order; when the last round would leave most workgroup
// slots idle its tiles are cut into 64 x 128 halves or 64 x 64 quarters.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "device_launch.hpp"
#include "k2_common.hpp"

namespace svdq {

namespace {

constexpr int NT = 256;             // threads per workgroup
constexpr int kBlk = 1024;          // one operand block: 64 lanes x 16 bytes
constexpr int kSxBlk = 128;         // activation scales of one 128-row band and group (floats)
constexpr int kWpBlk = 64;          // weight scale pairs of one 32-column strip and group (floats)
// LDS ring depth. Three stages (41,472 bytes) let three workgroups share a
// compute unit; four (55,296 bytes) leave room for two (three would need
// more than the 163,840 bytes of a compute unit's LDS).
constexpr int KSTAGES = 3;
constexpr int KAHEAD = KSTAGES - 1; // groups copied ahead of the one computed

// One group's operands for the whole tile (a 128 x 128 tile uses all of it).
struct alignas(16) TStage {
  uint8_t a[8][kBlk];               // activation operands of the tile's row blocks (int8 16q)
  uint8_t b[4][kBlk];               // 4-bit weight codes of the 4 waves' strips
  float sx[kSxBlk];                 // activation scales of the 128-row band
  float wp[4][kWpBlk];              // weight scale pairs of the 4 strips
};

#define LDSP(p) ((__attribute__((address_space(3))) void*)(p))


// Tile shapes: RB row blocks of 16 (every wave holds all of them) and CB
// column blocks of 16 per wave. 8 x 2: the 128 x 128 tile; 4 x 2 (64 x 128)
// and 4 x 1 (64 x 64): the pieces a thin last round is cut into.
template <int RB, int CB>
struct Shape {
  static constexpr int ROWS = 16 * RB;
  static constexpr int WCOLS = 16 * CB;             // columns per wave
  static constexpr int COLS = 4 * WCOLS;
  static constexpr int ACOPY = RB / 4;              // activation blocks each wave copies
  static constexpr int COPIES = ACOPY + 3;          // direct loads per wave and group
  static constexpr int NBLK = RB * CB;              // 16 x 16 blocks per wave
  // wait until the copies of the newest KAHEAD-1 groups are the only ones in flight
  static constexpr int WAIT_AHEAD = 0x0070 | (COPIES * (KAHEAD - 1));
  static_assert(COPIES * (KAHEAD - 1) < 16, "vmcnt field");
};
constexpr int kWaitAll = 0x0070;                    // vmcnt(0) lgkmcnt(0)
constexpr int kPartTile = 128 * 128;                // floats of one partial tile

template <int RB, int CB>
struct TScales {
  float sx[RB];                     // s_x of the lane's row per row block
  float ws[CB][4], wb[CB][4];       // (s_w/256, -12582912 s_w/256) of the lane's 4 columns per block
};

// t = P s_w exactly (see the file comment), then acc += t s_x with one
// rounding: the same value as P s_x s_w + acc rounded once.
template <int RB, int CB>
__device__ __forceinline__ void rescale(v4f& acc, const v4i& p, const TScales<RB, CB>& sc, int i,
                                        int j) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int pe = p[e];                     // scalar copy: see as_float()
    const float t = __builtin_fmaf(as_float(pe), sc.ws[j][e], sc.wb[j][e]);
    acc[e] = __builtin_fmaf(t, sc.sx[i], acc[e]);
  }
}

// The low-rank up-projection acc += fp16(D) . L2 for a wave whose region of Y
// starts at row m0 (16*RB rows) and column nw (16*CB columns), from the
// pre-kernel's fp16 D in operand order (D_t: per 16-row block and 32-rank
// chunk one 1 KB block; lane 16q + r holds row r, ranks 8q .. 8q+7), so an
// operand is one 16-byte load with nothing to convert. Work goes in units of
// 4 row blocks of one chunk; the next unit's loads are issued before this
// unit's matrix instructions. Every load is from a clamped in-bounds address;
// operands past R or M are zeroed after they arrive (selected, never
// multiplied in).
template <int RB, int CB>
__device__ __forceinline__ void lowrank_up_tiled(v4f (&acc)[RB][CB],
                                                 const uint16_t* __restrict__ Dt,
                                                 const uint16_t* __restrict__ L2t, int R,
                                                 int64_t M, int64_t N, int64_t m0, int64_t nw) {
  constexpr int NH = RB / 4;                        // units of 4 row blocks per chunk
  if (R <= 0) return;
  const int lane = threadIdx.x & 63;
  const int rl = lane & 15, q = lane >> 4;
  const int RC = (R + 31) / 32;
  const int NU = RC * NH;
  const int64_t Mb = (M + 15) / 16;
  const v8h zero = v8h{0, 0, 0, 0, 0, 0, 0, 0};
  auto load = [&](int u, v8h (&A)[4], v8h (&B)[CB]) {
    const int c = u / NH, h = u - c * NH;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t b = m0 / 16 + 4 * h + i;
      b = b < Mb ? b : Mb - 1;
      A[i] = *reinterpret_cast<const v8h*>(Dt + ((b * RC + c) * 64 + lane) * 8);
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int64_t n = nw + 16 * j + rl;
      const int kk = 32 * c + 8 * q;
      const bool ok = kk < R && n < N;
      B[j] = *reinterpret_cast<const v8h*>(L2t + (ok ? n * R + kk : 0));
    }
  };
  auto step = [&](int u, v8h (&A)[4], v8h (&B)[CB]) {
    const int c = u / NH, h = u - c * NH;
    const bool kval = 32 * c + 8 * q < R;
#pragma unroll
    for (int j = 0; j < CB; ++j) B[j] = (kval && nw + 16 * j + rl < N) ? B[j] : zero;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v8h a = (kval && m0 + 16 * (4 * h + i) + rl < M) ? A[i] : zero;
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        if (hh == h) {
#pragma unroll
          for (int j = 0; j < CB; ++j)
            acc[4 * hh + i][j] = mfma_f16_16x16x32(B[j], a, acc[4 * hh + i][j]);
        }
      }
    }
  };
  v8h A0[4], B0[CB], A1[4], B1[CB];
  load(0, A0, B0);
  // NU is the same for every lane, so loads past the last unit are skipped
  // by the whole wave
  for (int u = 0; u < NU; u += 2) {
    if (u + 1 < NU) load(u + 1, A1, B1);
    step(u, A0, B0);
    if (u + 1 >= NU) break;
    if (u + 2 < NU) load(u + 2, A0, B0);
    step(u + 1, A1, B1);
  }
}

// One tile of Y: rows m0 .. m0 + 16*RB - 1, columns n0 .. n0 + 64*CB - 1.
// PART: groups g_lo .. g_hi - 1 only, the low-rank term only when `lowrank`,
// and the fp32 sums go to `part` (16384 floats, lane order: block (i, j) of
// wave w at ((w*RB + i)*CB + j) * 256) for k2t_reduce_kernel; no epilogue.
template <int RB, int CB, bool Y_F16, bool GELU, bool PART = false>
__device__ __forceinline__ void tile_t(TStage (&st)[KSTAGES], const uint8_t* __restrict__ a_ops,
                                       const float* __restrict__ a_scales,
                                       const uint8_t* __restrict__ w_codes,
                                       const float* __restrict__ w_scales,
                                       const uint16_t* __restrict__ Dt,
                                       const uint16_t* __restrict__ L2t, int R,
                                       const float* __restrict__ bias, void* __restrict__ Y,
                                       int64_t M, int64_t N, int64_t K, int64_t ldy, int64_t m0,
                                       int64_t n0, int g_lo = 0, int g_hi = -1,
                                       bool lowrank = true, float* __restrict__ part = nullptr) {
  using S = Shape<RB, CB>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int rl = lane & 15, q = lane >> 4;
  const int G = static_cast<int>(K / kGroup);
  const int g_first = g_lo, g_end = g_hi < 0 ? G : g_hi;   // this tile's groups
  const int64_t Mb = (M + 15) / 16, Ns = (N + 31) / 32;
  const int64_t nw = n0 + S::WCOLS * wave;          // the wave's first column
  const int rb0 = static_cast<int>((m0 % 128) / 16);   // the tile's first row block in its band
  const int rs = (S::WCOLS * wave) / 32;            // the wave's strip among the 4 copied
  const int hb = CB == 1 ? static_cast<int>((nw / 16) & 1) : 0;   // its half of that strip
  // this wave's copies: activation row blocks ACOPY*w .. +ACOPY-1 of the tile
  // (clamped to the last row block: their outputs are never stored), the
  // strip holding its columns and that strip's scale pairs, and half of the
  // band's activation scales. Every wave issues the same number of copies.
  // Bases are wave-uniform; each lane adds a 32-bit offset.
  auto clamp_b = [&](int64_t b) { return b < Mb ? b : Mb - 1; };
  auto clamp_s = [&](int64_t s) { return s < Ns ? s : Ns - 1; };
  const uint8_t* ga[S::ACOPY];
#pragma unroll
  for (int c = 0; c < S::ACOPY; ++c)
    ga[c] = a_ops + clamp_b(m0 / 16 + S::ACOPY * wave + c) * G * kBlk;
  const uint8_t* gb = w_codes + clamp_s(nw / 32) * G * kBlk;
  const float* gx = a_scales + (m0 / 128) * G * kSxBlk + 64 * (wave & 1);
  const float* gw = w_scales + clamp_s(nw / 32) * G * kWpBlk;
  const uint32_t lo16 = 16u * static_cast<uint32_t>(lane);
  const uint32_t lo4 = 4u * static_cast<uint32_t>(lane);

  auto copy = [&](TStage& s, int g) {
    g = g < g_end ? g : g_end - 1;
    const int64_t o = static_cast<int64_t>(g) * kBlk;
#pragma unroll
    for (int c = 0; c < S::ACOPY; ++c)
      __builtin_amdgcn_global_load_lds(ga[c] + o + lo16, LDSP(&s.a[S::ACOPY * wave + c][0]), 16, 0,
                                       0);
    __builtin_amdgcn_global_load_lds(gb + o + lo16, LDSP(&s.b[wave][0]), 16, 0, 0);
    // half of the band's activation scales (waves 2 and 3 write the same
    // bytes as waves 0 and 1: a direct-to-LDS load of fewer than 4 bytes per
    // lane still takes a 4-byte LDS slot per lane, so a quarter per wave
    // would need 2-byte slots, which do not exist)
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<const uint8_t*>(gx + static_cast<int64_t>(g) * kSxBlk) + lo4,
        LDSP(&s.sx[64 * (wave & 1)]), 4, 0, 0);
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<const uint8_t*>(gw + static_cast<int64_t>(g) * kWpBlk) + lo4,
        LDSP(&s.wp[rs][0]), 4, 0, 0);
  };
  auto read_a = [&](const TStage& s, int i) {
    return *reinterpret_cast<const v4i*>(&s.a[i][16 * lane]);
  };

#pragma unroll
  for (int c = 0; c < KAHEAD; ++c) copy(st[c], g_first + c);

  // the low-rank branch starts the accumulators while the first groups copy
  v4f acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  if (!PART || lowrank) lowrank_up_tiled<RB, CB>(acc, Dt, L2t, R, M, N, m0, nw);

  // Iteration g computes group g from stage g % KSTAGES. Its barrier follows
  // this wave's wait for its own copies of group g, so after it every copy of
  // group g has landed and every wave is done with group g-1, whose stage then
  // takes group g+KAHEAD. Inside the group the matrix instructions of row
  // block i go out before the rescale of row block i-1, so the partials of
  // only two row blocks are live (and two activation operands), which keeps
  // the kernel at three waves per SIMD.
  const v4i seed = v4i{kMagicSeed, kMagicSeed, kMagicSeed, kMagicSeed};
  int sg = 0, sp = KSTAGES - 1;                 // stages of groups g and g-1
  for (int g = g_first; g < g_end; ++g) {
    const TStage& s = st[sg];
    __builtin_amdgcn_s_waitcnt(S::WAIT_AHEAD);
    __builtin_amdgcn_s_barrier();
    copy(st[sp], g + KAHEAD);                   // group g-1's stage takes group g+KAHEAD
    sp = sg;
    sg = sg + 1 == KSTAGES ? 0 : sg + 1;

    const uint4 braw = *reinterpret_cast<const uint4*>(&s.b[wave][16 * lane]);
    v4i A[2];
    A[0] = read_a(s, 0);
    TScales<RB, CB> sc;
    // activation scales: row block i of the band, row r, at 64 (i/4) + 4r + i%4
    // (the 16 rows' float4 of one instruction are 256 contiguous bytes)
#pragma unroll
    for (int h = 0; h < RB / 4; ++h) {
      const float4 v = *reinterpret_cast<const float4*>(&s.sx[64 * (rb0 / 4 + h) + 4 * rl]);
      sc.sx[4 * h] = v.x;
      sc.sx[4 * h + 1] = v.y;
      sc.sx[4 * h + 2] = v.z;
      sc.sx[4 * h + 3] = v.w;
    }
    // weight pairs: column 16j + 4q + e of the strip at 16q + 8j + 2e
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int jj = CB == 2 ? j : hb;
      const float4 u = *reinterpret_cast<const float4*>(&s.wp[rs][16 * q + 8 * jj]);
      const float4 v = *reinterpret_cast<const float4*>(&s.wp[rs][16 * q + 8 * jj + 4]);
      sc.ws[j][0] = u.x;
      sc.wb[j][0] = u.y;
      sc.ws[j][1] = u.z;
      sc.wb[j][1] = u.w;
      sc.ws[j][2] = v.x;
      sc.wb[j][2] = v.y;
      sc.ws[j][3] = v.z;
      sc.wb[j][3] = v.w;
    }
    v4i B[CB];
    if constexpr (CB == 2) {
      B[0] = widen_codes(make_uint2(braw.x, braw.y));
      B[1] = widen_codes(make_uint2(braw.z, braw.w));
    } else {
      B[0] = widen_codes(hb ? make_uint2(braw.z, braw.w) : make_uint2(braw.x, braw.y));
    }
    v4i P[2][CB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (i + 1 < RB) A[(i + 1) & 1] = read_a(s, i + 1);
#pragma unroll
      for (int j = 0; j < CB; ++j) P[i & 1][j] = mfma_i8_16x16x64(B[j], A[i & 1], seed);
      if (i > 0) {
#pragma unroll
        for (int j = 0; j < CB; ++j) rescale(acc[i - 1][j], P[(i - 1) & 1][j], sc, i - 1, j);
      }
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) rescale(acc[RB - 1][j], P[(RB - 1) & 1][j], sc, RB - 1, j);
  }

  // copies of groups past the end land in stages nobody reads; wait for them
  // before the LDS is used for the output
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __builtin_amdgcn_s_barrier();
  if constexpr (PART) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j)
        *reinterpret_cast<v4f*>(part + (((wave * RB + i) * CB + j) * 64 + lane) * 4) = acc[i][j];
    return;
  }
  if constexpr (Y_F16 && RB == 8 && CB == 2) {
    static_assert(sizeof(TStage) * KSTAGES >= 128 * 256, "a 128 x 128 fp16 tile in LDS");
    if (m0 + 128 <= M && n0 + 128 <= N &&
        ((reinterpret_cast<uintptr_t>(Y) | static_cast<uintptr_t>(ldy * 2)) % 16) == 0) {
      // the whole tile through LDS: 128 rows of 256 bytes, the 16-byte
      // units of row r XOR-swizzled by r % 16; then every store instruction
      // writes 4 rows of 256 bytes (8 whole cache lines)
      uint8_t* lds = reinterpret_cast<uint8_t*>(&st[0]);
      float bv[CB][4];
#pragma unroll
      for (int j = 0; j < CB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bv[j][e] = bias != nullptr ? bias[nw + 16 * j + 4 * q + e] : 0.f;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int row = 16 * i + rl;
#pragma unroll
        for (int j = 0; j < CB; ++j) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = acc[i][j][e] + bv[j][e];
            if constexpr (GELU) v[e] = gelu_tanh_f32(v[e]);
          }
          const uint32_t lo = static_cast<uint32_t>(f2h(v[0])) | (static_cast<uint32_t>(f2h(v[1])) << 16);
          const uint32_t hi = static_cast<uint32_t>(f2h(v[2])) | (static_cast<uint32_t>(f2h(v[3])) << 16);
          const int unit = 4 * wave + 2 * j + (q >> 1);     // 16-byte unit of the 4 columns
          *reinterpret_cast<uint2*>(lds + row * 256 + ((unit ^ (row & 15)) << 4) + ((q & 1) << 3)) =
              make_uint2(lo, hi);
        }
      }
      __syncthreads();
      _Float16* Yh = static_cast<_Float16*>(Y);
      const int u = lane & 15, r4 = lane >> 4;
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = 32 * wave + 4 * it + r4;
        const uint4 v = *reinterpret_cast<const uint4*>(lds + row * 256 + ((u ^ (row & 15)) << 4));
        *reinterpret_cast<uint4*>(Yh + (m0 + row) * ldy + n0 + 8 * u) = v;
      }
      return;
    }
  }
  bias_store_at<16 * RB, 16 * CB, Y_F16, GELU>(acc, bias, Y, M, N, ldy, m0, nw);
}

// Workgroups 0 .. n_full-1 take the first n_full 128 x 128 tiles of the
// banded order; the rest take the remaining tiles in `split` pieces (2: 64 x
// 128 halves, 4: 64 x 64 quarters). A piece wholly outside Y returns at once
// (the same for every wave of the workgroup, before any barrier).
// PART: split along K. Every tile is taken by `split` workgroups, slice s
// computing groups s*G/split .. (s+1)*G/split - 1 (slice 0 with the low-rank
// term) into its fp32 partial tile in `partial`; k2t_reduce_kernel finishes Y.
template <bool Y_F16, bool GELU, bool PART = false>
__global__ __launch_bounds__(NT, 3) void k2t_w4a4_kernel(
    const uint8_t* __restrict__ a_ops, const float* __restrict__ a_scales,
    const uint8_t* __restrict__ w_codes, const float* __restrict__ w_scales,
    const uint16_t* __restrict__ Dt, const uint16_t* __restrict__ L2t, int R,
    const float* __restrict__ bias, void* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int tiles_m, int tiles_n, int n_full, int split, float* __restrict__ partial) {
  __shared__ TStage st[KSTAGES];
  const int b = static_cast<int>(blockIdx.x);
  int tm, tn;
  if constexpr (PART) {
    const int T = tiles_m * tiles_n;
    const int unit = xcd_contiguous(b, T * split);
    const int tile = unit / split, slice = unit - tile * split;
    banded_tile(tile, tiles_m, tiles_n, tm, tn);
    const int G = static_cast<int>(K / kGroup);
    tile_t<8, 2, Y_F16, GELU, true>(st, a_ops, a_scales, w_codes, w_scales, Dt, L2t, R, bias, Y, M,
                                    N, K, ldy, static_cast<int64_t>(tm) * 128,
                                    static_cast<int64_t>(tn) * 128, slice * G / split,
                                    (slice + 1) * G / split, slice == 0,
                                    partial + (static_cast<int64_t>(slice) * T + tile) * kPartTile);
    return;
  } else {
    if (b < n_full) {
      banded_tile(xcd_contiguous(b, n_full), tiles_m, tiles_n, tm, tn);
      tile_t<8, 2, Y_F16, GELU>(st, a_ops, a_scales, w_codes, w_scales, Dt, L2t, R, bias, Y, M, N,
                                K, ldy, static_cast<int64_t>(tm) * 128,
                                static_cast<int64_t>(tn) * 128);
      return;
    }
    const int u = b - n_full;
    banded_tile(n_full + u / split, tiles_m, tiles_n, tm, tn);
    const int part = u % split;
    const int64_t m0 = static_cast<int64_t>(tm) * 128 + 64 * (split == 2 ? part : part >> 1);
    const int64_t n0 = static_cast<int64_t>(tn) * 128 + (split == 4 ? 64 * (part & 1) : 0);
    if (m0 >= M || n0 >= N) return;
    if (split == 2)
      tile_t<4, 2, Y_F16, GELU>(st, a_ops, a_scales, w_codes, w_scales, Dt, L2t, R, bias, Y, M, N,
                                K, ldy, m0, n0);
    else
      tile_t<4, 1, Y_F16, GELU>(st, a_ops, a_scales, w_codes, w_scales, Dt, L2t, R, bias, Y, M, N,
                                K, ldy, m0, n0);
  }
}

// Y from the partial tiles of the split kernel: the S slices summed in slice
// order, then bias, the activation and one rounding, as the unsplit
// epilogue does. One thread per 4 consecutive outputs (a lane's float4).
template <bool Y_F16, bool GELU>
__global__ __launch_bounds__(256) void k2t_reduce_kernel(const float* __restrict__ part, int S,
                                                         int T, int tiles_m, int tiles_n,
                                                         const float* __restrict__ bias,
                                                         void* __restrict__ Y, int64_t M,
                                                         int64_t N, int64_t ldy) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= static_cast<int64_t>(T) * (kPartTile / 4)) return;
  const int tile = static_cast<int>(t / (kPartTile / 4));
  const int r = static_cast<int>(t - static_cast<int64_t>(tile) * (kPartTile / 4));
  const int lane = r & 63, blk = r >> 6;             // blk = (wave*8 + i)*2 + j
  const int j = blk & 1, i = (blk >> 1) & 7, w = blk >> 4;
  int tm, tn;
  banded_tile(tile, tiles_m, tiles_n, tm, tn);
  const int64_t m = static_cast<int64_t>(tm) * 128 + 16 * i + (lane & 15);
  const int64_t n = static_cast<int64_t>(tn) * 128 + 32 * w + 16 * j + 4 * (lane >> 4);
  if (m >= M || n >= N) return;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sl = 0; sl < S; ++sl) {
    const float4 p = *reinterpret_cast<const float4*>(
        part + ((static_cast<int64_t>(sl) * T + tile) * (kPartTile / 4) + r) * 4);
    v[0] += p.x;
    v[1] += p.y;
    v[2] += p.z;
    v[3] += p.w;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (n + e >= N) break;
    float y = v[e] + (bias != nullptr ? bias[n + e] : 0.f);
    if constexpr (GELU) y = gelu_tanh_f32(y);
    if constexpr (Y_F16)
      static_cast<uint16_t*>(Y)[m * ldy + n + e] = f2h(y);
    else
      static_cast<float*>(Y)[m * ldy + n + e] = y;
  }
}

// Workgroups of this kernel resident at once on the current device (compute
// units times the occupancy its registers and LDS allow), cached per device.
int k2t_slots() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return resident_slots();
  if (cache[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0 ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(k2t_w4a4_kernel<true, false>), NT, 0) !=
            hipSuccess ||
        per_cu <= 0)
      return resident_slots();
    cache[dev] = cus * per_cu;
  }
  return cache[dev];
}

}  // namespace

// Split along K when the tiles fill at most a quarter of the resident
// workgroup slots and the rows hold at least 32 groups (the UNet's 32x32
// convolution: 160 tiles for 768 slots, each running 180 groups in series):
// `split` = slots / tiles, at most G / 16 and 8, so that the slices about
// fill the slots. The partial tiles cost a pass over S x 64 KB per tile;
// measured on MI355X inside the step, the 32x32 convolution's GEMM took 60.6
// against 75.5 us split in 4, the 64x64 one (320 tiles, 90 groups) 66.8
// against 56.5 us split in 2, hence the quarter.
int k2t_ksplit(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < kGroup) return 1;
  const int64_t T = ((M + 127) / 128) * ((N + 127) / 128), slots = k2t_slots(), G = K / kGroup;
  if (4 * T > slots || G < 32) return 1;
  int64_t S = slots / T;
  if (S > G / 16) S = G / 16;
  if (S > 8) S = 8;
  return S < 2 ? 1 : static_cast<int>(S);
}

size_t k2t_split_bytes(int64_t M, int64_t N, int64_t K) {
  const int S = k2t_ksplit(M, N, K);
  if (S == 1) return 0;
  const int64_t T = ((M + 127) / 128) * ((N + 127) / 128);
  return static_cast<size_t>(S) * static_cast<size_t>(T) * kPartTile * 4;
}

hipError_t launch_k2t(const uint8_t* a_ops, const float* a_scales, const uint8_t* w_codes_t,
                      const float* w_scales_t, const uint16_t* Dt, const uint16_t* L2t, int R,
                      const float* bias, void* Y, bool y_f16, int64_t M, int64_t N, int64_t K,
                      int64_t ldy, bool gelu, hipStream_t stream, float* part) {
  const int tiles_m = static_cast<int>((M + 127) / 128);
  const int tiles_n = static_cast<int>((N + 127) / 128);
  const int T = tiles_m * tiles_n;
  const int KS = part != nullptr ? k2t_ksplit(M, N, K) : 1;
  if (KS > 1) {
    const dim3 grid(static_cast<unsigned>(T * KS)), block(NT);
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, grid, block, 0, stream, a_ops, a_scales, w_codes_t, w_scales_t,
                         Dt, L2t, R, bias, Y, M, N, K, ldy, tiles_m, tiles_n, 0, KS, part);
    };
    auto red = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(T * (kPartTile / 4 / 256))),
                         dim3(256), 0, stream, part, KS, T, tiles_m, tiles_n, bias, Y, M, N, ldy);
    };
    if (y_f16)
      gelu ? go(k2t_w4a4_kernel<true, true, true>) : go(k2t_w4a4_kernel<true, false, true>);
    else
      gelu ? go(k2t_w4a4_kernel<false, true, true>) : go(k2t_w4a4_kernel<false, false, true>);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    if (y_f16)
      gelu ? red(k2t_reduce_kernel<true, true>) : red(k2t_reduce_kernel<true, false>);
    else
      gelu ? red(k2t_reduce_kernel<false, true>) : red(k2t_reduce_kernel<false, false>);
    return hipGetLastError();
  }
  // the tiles of a thin last round are cut into halves or quarters, so that
  // they fill more of the resident workgroup slots
  const int S = k2t_slots();
  const int left = T < S ? T : T % S;
  const int split = (left > 0 && 4 * left <= S) ? 4 : (left > 0 && 2 * left <= S) ? 2 : 1;
  const int n_split = split > 1 ? left : 0;
  const int n_full = T - n_split;
  const dim3 grid(static_cast<unsigned>(n_full + split * n_split)), block(NT);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, a_ops, a_scales, w_codes_t, w_scales_t, Dt,
                       L2t, R, bias, Y, M, N, K, ldy, tiles_m, tiles_n, n_full, split, nullptr);
  };
  if (y_f16)
    gelu ? go(k2t_w4a4_kernel<true, true>) : go(k2t_w4a4_kernel<true, false>);
  else
    gelu ? go(k2t_w4a4_kernel<false, true>) : go(k2t_w4a4_kernel<false, false>);
  return hipGetLastError();
}

}  // namespace svdq
