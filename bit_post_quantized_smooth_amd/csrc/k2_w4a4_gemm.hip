// K2: the W4A4 GEMM of the SVDQuant linear layer with the low-rank
// up-projection and the bias fused in (gfx950).
//
// Both operands are 4-bit (SVDQuant abstract: weights and activations at
// 4 bits; chattools.cn overview, section "SVDQuant的主要功能", quantization
// item). gfx950 has no 4-bit integer matrix instruction, so the nibbles are
// widened to int8 lanes holding 16*q (two bit operations per 4 codes, see
// device_common.hpp) and fed to v_mfma_i32_16x16x64_i8: one instruction covers
// exactly one 64-channel group of a 16 x 16 output block, so its int32 result
// is the exact group partial (times 256).
//
// Per-group rescale: the int32 accumulator is seeded with the bit pattern of
// 1.5*2^23, so the partial reads back as the float f = 12582912 + 256 P. Then
//     t   = fma(f, s_x, -12582912 s_x)  = 256 P s_x   (exact: |P| <= 64*49, so
//                                                       256 P s_x fits in 24 bits)
//     acc = fma(t, s_w, acc)                            (the one rounding)
// i.e. two fp32 ops per output and group, the second reading the fp16 weight
// scale directly (v_fma_mix_f32); the factor 256 is removed once after the K
// loop. These two ops per output and group, not the matrix instruction, bound
// the kernel: one v_mfma_i32_16x16x64_i8 does the integer work of 256 outputs
// x 1 group in about the time of 4 wave-wide fp32 ops.
//
// The low-rank branch (the Nunchaku engine fuses it into the low-bit kernel:
// SVDQuant abstract; the disruptive-concepts.com post, section "Nunchaku:
// Fusing Precision and Speed") runs after the K loop as fp16 MFMAs on the same
// fp32 accumulators: acc += fp16(D) . L2, then the bias, optionally the GELU
// of a DiT MLP's first layer (fused so the intermediate is written once), then
// one rounding to the output type.
//
// Tiling: a 256-thread workgroup computes a square tile of Y; each of its 4
// waves owns a WT x WT quarter of it (WT/16 x WT/16 blocks of 16 x 16). The
// matrix instruction takes the weight fragment as its first operand, so a lane
// ends up holding 4 consecutive columns of one row of each block (a full
// quarter of an fp16 Y goes out through the then idle LDS in whole cache
// lines, any other in 8-byte stores). The K loop stages one group at a time through
// double-buffered LDS; the loader widens the codes once, as it stores them, in
// operand order: the 16 bytes a lane feeds to the matrix instruction for
// (row block, group) sit at [buffer][row block][lane], so each operand is one
// contiguous 16-byte LDS read per lane; it also converts each activation scale
// to fp32 once, next to -1.5*2^23 times it. The next group's operands are read
// while the current group computes.
//
// Most tiles are 128 x 128 (WT = 64). When the last round of tiles would
// leave most of the chip idle (leftover tiles filling at most a quarter of the
// resident workgroup slots), the leftover tiles are cut into 64 x 64 tiles
// (WT = 32) in the same launch, so the tail takes about a quarter of a round. Every output
// element goes through the same arithmetic in either size.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "device_launch.hpp"
#include "k2_common.hpp"

namespace svdq {

namespace {

constexpr int NT = 256;             // threads per workgroup

template <int WT>
struct TileCfg {
  static constexpr int BT = 2 * WT;         // tile edge
  static constexpr int NB = WT / 16;        // 16 x 16 blocks per wave edge
};

template <int WT>
struct Smem {
  v4i a[2][2 * WT / 16][64];        // widened A operands of one group [buf][row block][lane]
  v4i b[2][2 * WT / 16][64];        // widened B operands
  float sx[2][2][16][WT / 16];      // activation scales [buf][row/WT][row%16][(row%WT)/16], fp32
  float be[2][2][16][WT / 16];      // -12582912 * each activation scale, same layout
                                    // (converted once by the loader, not by every wave)
  uint16_t sw[2][2 * WT];           // weight scales [buf][col]
};

// LDS slot of operand entry e = q*16 + row: entries of chunks q = 2, 3 are
// swapped in blocks of 4 (XOR 12). The two threads of a row store chunks q and
// q+2 side by side; without the swap those two 16-byte stores fall on the same
// banks. Reads stay one permutation of 8 (or 16) consecutive slots per lane
// group, so they remain conflict-free.
__device__ __forceinline__ int swz(int e) { return e ^ ((e >> 5) * 12); }

// One group's slice of the tile, staged in registers between its global load
// and its widened store to LDS. A group of a tile is 2*BT rows (BT of A, BT of
// B) of 32 bytes, loaded as 16-byte halves: for BT = 128 thread t loads half
// t%2 of A row t/2 and of B row t/2; for BT = 64 threads 0..127 load A rows,
// threads 128..255 B rows. Threads 0..BT-1 also load an A row scale and
// threads BT..2BT-1 a B column scale (for BT = 64 the others load a scale they
// do not store). Rows and columns past M or N are clamped to the last one:
// their results are computed but never stored, so every load is
// unconditional and in bounds.
template <int WT>
struct Loader {
  static constexpr int BT = TileCfg<WT>::BT;
  static constexpr int NC = BT == 128 ? 2 : 1;      // 16-byte chunks per thread
  const uint8_t* row[NC];
  const uint16_t* sc_row;
  uint4 c[NC];
  uint16_t sc;

  __device__ __forceinline__ void init(const uint8_t* a_codes, const uint16_t* a_scales,
                                       const uint8_t* w_codes, const uint16_t* w_scales,
                                       int64_t m0, int64_t n0, int64_t M, int64_t N, int64_t K) {
    const int t = threadIdx.x;
    const int64_t kb = K / 2, G = K / kGroup;
    auto clamp_m = [&](int64_t r) { return m0 + r < M ? m0 + r : M - 1; };
    auto clamp_n = [&](int64_t r) { return n0 + r < N ? n0 + r : N - 1; };
    if constexpr (BT == 128) {
      row[0] = a_codes + clamp_m(t >> 1) * kb + 16 * (t & 1);
      row[1] = w_codes + clamp_n(t >> 1) * kb + 16 * (t & 1);
    } else {
      const int r = (t & 127) >> 1;
      row[0] = (t < 128 ? a_codes + clamp_m(r) * kb : w_codes + clamp_n(r) * kb) + 16 * (t & 1);
    }
    const int s = t < 2 * BT ? t : 0;
    sc_row = s < BT ? a_scales + clamp_m(s) * G : w_scales + clamp_n(s - BT) * G;
  }

  __device__ __forceinline__ void load(int64_t g) {
#pragma unroll
    for (int i = 0; i < NC; ++i) c[i] = *reinterpret_cast<const uint4*>(row[i] + g * kGroupBytes);
    sc = sc_row[g];
  }

  // Widen and store: the 16 bytes of row r hold chunks q = 2h, 2h+1 (codes
  // 16q .. 16q+15), which go to lane q*16 + r%16 of row block r/16.
  __device__ __forceinline__ void store(Smem<WT>& sm, int buf) const {
    const int t = threadIdx.x;
    const int h = t & 1;
    const int r = (BT == 128 ? t : (t & 127)) >> 1;
    const int rb = r >> 4, rr = r & 15;
    const int e0 = swz((2 * h) * 16 + rr), e1 = swz((2 * h + 1) * 16 + rr);
    if constexpr (BT == 128) {
      sm.a[buf][rb][e0] = widen_codes(make_uint2(c[0].x, c[0].y));
      sm.a[buf][rb][e1] = widen_codes(make_uint2(c[0].z, c[0].w));
      sm.b[buf][rb][e0] = widen_codes(make_uint2(c[1].x, c[1].y));
      sm.b[buf][rb][e1] = widen_codes(make_uint2(c[1].z, c[1].w));
    } else {
      v4i(*dst)[64] = t < 128 ? sm.a[buf] : sm.b[buf];
      dst[rb][e0] = widen_codes(make_uint2(c[0].x, c[0].y));
      dst[rb][e1] = widen_codes(make_uint2(c[0].z, c[0].w));
    }
    if (t < BT) {
      const float sxf = h2f(sc);
      sm.sx[buf][t / WT][t & 15][(t % WT) >> 4] = sxf;
      sm.be[buf][t / WT][t & 15][(t % WT) >> 4] = sxf * -kMagicF;   // exact: 3 * 2^22 * s_x
    }
    else if (t < 2 * BT)
      sm.sw[buf][t - BT] = sc;
  }
};

// Operands and scales of one group for one wave.
template <int NB>
struct Frags {
  v4i A[NB], B[NB];
};
template <int NB>
struct Scales {
  float sx[NB];                     // activation scale of the lane's row, per row block
  float be[NB];                     // -12582912 * sx
  uint2 swp[NB];                    // fp16 weight scales of the lane's 4 columns, per column block
};

template <int WT>
__device__ __forceinline__ void read_frags(Frags<WT / 16>& f, const Smem<WT>& sm, int buf, int wm,
                                           int wn, int lane) {
  constexpr int NB = WT / 16;
  const int sl = swz(lane);
#pragma unroll
  for (int i = 0; i < NB; ++i) f.A[i] = sm.a[buf][wm * NB + i][sl];
#pragma unroll
  for (int j = 0; j < NB; ++j) f.B[j] = sm.b[buf][wn * NB + j][sl];
}

template <int WT>
__device__ __forceinline__ void read_scales(Scales<WT / 16>& sc, const Smem<WT>& sm, int buf,
                                            int wm, int wn, int lane) {
  constexpr int NB = WT / 16;
  const int q = lane >> 4, rl = lane & 15;
#pragma unroll
  for (int j = 0; j < NB; ++j)
    sc.swp[j] = *reinterpret_cast<const uint2*>(&sm.sw[buf][wn * WT + j * 16 + 4 * q]);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    sc.sx[i] = sm.sx[buf][wm][rl][i];
    sc.be[i] = sm.be[buf][wm][rl][i];
  }
}

template <int NB>
__device__ __forceinline__ float sw_of(const Scales<NB>& sc, int j, int e) {
  const uint32_t w = (e < 2) ? sc.swp[j].x : sc.swp[j].y;
  return h2f(static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xFFFFu)));
}

// Rescale of one 16 x 16 block of group g (two fp32 ops per output):
//   t = (12582912 + 256 P) s_x - 12582912 s_x = 256 P s_x (exact); acc += t s_w
template <int NB>
__device__ __forceinline__ void rescale_block(v4f& acc, const v4i& p, const Scales<NB>& sc,
                                              int i, int j) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int pe = p[e];                     // scalar copy: see as_float()
    const float t = __builtin_fmaf(as_float(pe), sc.sx[i], sc.be[i]);
    acc[e] = __builtin_fmaf(t, sw_of(sc, j, e), acc[e]);
  }
}

// One tile of Y: rows m0 .. m0 + 2*WT - 1, columns n0 .. n0 + 2*WT - 1.
template <int WT, bool Y_F16, bool GELU>
__device__ __forceinline__ void gemm_tile(
    Smem<WT>& sm, const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
    const uint8_t* __restrict__ w_codes, const uint16_t* __restrict__ w_scales,
    const float* __restrict__ D, const uint16_t* __restrict__ L2t, int R,
    const float* __restrict__ bias, void* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int64_t m0, int64_t n0) {
  constexpr int NB = WT / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t G = K / kGroup;
  const v4i seed = v4i{kMagicSeed, kMagicSeed, kMagicSeed, kMagicSeed};

  v4f acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Software pipeline over the 64-channel groups. Iteration g rescales the
  // integer partials P of group g block by block and, right after each block,
  // issues the matrix instruction of group g+1 into the same registers, so the
  // matrix core and the vector ALU work side by side within the wave. LDS
  // holds two groups; a thread's registers hold the next group's codes between
  // their global load and their widened store.
  Loader<WT> ld;
  ld.init(a_codes, a_scales, w_codes, w_scales, m0, n0, M, N, K);
  ld.load(0);
  ld.store(sm, 0);
  if (G > 1) {
    ld.load(1);
    ld.store(sm, 1);
  }
  if (G > 2) ld.load(2);
  __syncthreads();

  v4i P[NB][NB];
  Frags<NB> f;
  Scales<NB> cur;
  read_frags<WT>(f, sm, 0, wm, wn, lane);
  read_scales<WT>(cur, sm, 0, wm, wn, lane);
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) P[i][j] = mfma_i8_16x16x64(f.B[j], f.A[i], seed);

  for (int64_t g = 0; g + 1 < G; ++g) {
    const int buf = static_cast<int>(g & 1);
    __syncthreads();                 // all waves are done reading group g's buffer; group g+1 is stored
    if (g + 2 < G) {
      ld.store(sm, buf);             // group g+2 replaces group g
      if (g + 3 < G) ld.load(g + 3);
    }
    read_frags<WT>(f, sm, buf ^ 1, wm, wn, lane);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        rescale_block(acc[i][j], P[i][j], cur, i, j);
        P[i][j] = mfma_i8_16x16x64(f.B[j], f.A[i], seed);
      }
    }
    // keep the schedule interleaved: 8 vector ops (one block's rescale), then
    // one matrix instruction, for every block
#pragma unroll
    for (int b = 0; b < NB * NB; ++b) {
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // group g+1's scales, read into the same registers once group g's are
    // used up (no second set, no copies at the end of the iteration; the
    // barrier ahead of the next iteration's stores waits for these reads)
    read_scales<WT>(cur, sm, buf ^ 1, wm, wn, lane);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) rescale_block(acc[i][j], P[i][j], cur, i, j);

  // the group sums carry the factor 256 of the widened operands: remove it (exact)
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] *= 0.00390625f;

  lowrank_up<WT, WT>(acc, D, L2t, R, M, N, m0, n0);
  if constexpr (Y_F16 && WT == 64) {
    static_assert(sizeof(Smem<WT>) >= 4 * WT * 128, "each wave stages a WT x 64 fp16 tile");
    __syncthreads();                 // every wave is done reading the operands in LDS
    if (lds_store_ok<WT, WT>(Y, ldy, M, N, m0, n0)) {
      bias_store_lds_f16<WT, WT, GELU>(acc, bias, static_cast<_Float16*>(Y), ldy, m0, n0,
                                       reinterpret_cast<uint8_t*>(&sm) + wave * WT * 128);
      return;
    }
  }
  bias_store<WT, WT, Y_F16, GELU>(acc, bias, Y, M, N, ldy, m0, n0);
}

// Workgroups 0 .. n_full-1 take the first n_full 128 x 128 tiles of the banded
// order; the remaining workgroups take the leftover tiles in quarters.
template <bool Y_F16, bool GELU>
__global__ __launch_bounds__(NT, 2) void k2_w4a4_kernel(
    const uint8_t* __restrict__ a_codes, const uint16_t* __restrict__ a_scales,
    const uint8_t* __restrict__ w_codes, const uint16_t* __restrict__ w_scales,
    const float* __restrict__ D, const uint16_t* __restrict__ L2t, int R,
    const float* __restrict__ bias, void* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int tiles_m, int tiles_n, int n_full) {
  __shared__ union {
    Smem<64> full;
    Smem<32> quarter;
  } sm;
  const int b = static_cast<int>(blockIdx.x);
  int tm, tn;
  if (b < n_full) {
    banded_tile(xcd_contiguous(b, n_full), tiles_m, tiles_n, tm, tn);
    gemm_tile<64, Y_F16, GELU>(sm.full, a_codes, a_scales, w_codes, w_scales, D, L2t, R, bias, Y, M,
                         N, K, ldy, static_cast<int64_t>(tm) * 128,
                         static_cast<int64_t>(tn) * 128);
  } else {
    const int qb = b - n_full;
    const int quarter = qb & 3;
    banded_tile(n_full + (qb >> 2), tiles_m, tiles_n, tm, tn);
    gemm_tile<32, Y_F16, GELU>(sm.quarter, a_codes, a_scales, w_codes, w_scales, D, L2t, R, bias, Y,
                         M, N, K, ldy, static_cast<int64_t>(tm) * 128 + 64 * (quarter >> 1),
                         static_cast<int64_t>(tn) * 128 + 64 * (quarter & 1));
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
      const int pe = r[e];
      if (mr < rows && nb < N) P[(mr * N + nb) * G + g] = pe >> 8;   // 256 P -> P, exact
    }
  }
}

}  // namespace

// Resident workgroup slots of the device (2 per compute unit), cached per device.
int resident_slots() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev] = 2 * cus;
  }
  return cache[dev];
}

hipError_t launch_k2(const uint8_t* a_codes, const uint16_t* a_scales, const uint8_t* w_codes,
                     const uint16_t* w_scales, const float* D, const uint16_t* L2t, int R,
                     const float* bias, void* Y, bool y_f16, int64_t M, int64_t N, int64_t K,
                     int64_t ldy, bool gelu, hipStream_t stream) {
  const int tiles_m = static_cast<int>((M + 127) / 128);
  const int tiles_n = static_cast<int>((N + 127) / 128);
  const int T = tiles_m * tiles_n;
  // leftover tiles of the last round; quartered when they would fill at most
  // a quarter of the resident slots (measured: with more of them, whole tiles,
  // one per compute unit, finish sooner than four times as many quarters)
  const int S = resident_slots();
  const int left = T < S ? T : T % S;
  const int n_quarter_tiles = (left > 0 && 4 * left <= S) ? left : 0;
  const int n_full = T - n_quarter_tiles;
  const dim3 grid(static_cast<unsigned>(n_full + 4 * n_quarter_tiles)), block(NT);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, a_codes, a_scales, w_codes, w_scales, D,
                       L2t, R, bias, Y, M, N, K, ldy, tiles_m, tiles_n, n_full);
  };
  if (y_f16)
    gelu ? go(k2_w4a4_kernel<true, true>) : go(k2_w4a4_kernel<true, false>);
  else
    gelu ? go(k2_w4a4_kernel<false, true>) : go(k2_w4a4_kernel<false, false>);
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
