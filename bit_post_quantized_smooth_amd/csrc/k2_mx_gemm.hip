// K2-MX: the 4-bit GEMM of the SVDQuant linear layer in the MXFP4 format,
// with the low-rank up-projection and the bias fused in (gfx950).
//
// The pages name a 4-bit floating-point version of the method for the newest
// hardware of one vendor (taicenter.com news page on SVDQuant, section on
// hardware co-design for Blackwell GPUs, NVFP4 item). On CDNA4 the matching
// format is OCP MXFP4: E2M1 values with one E8M0 power-of-two scale per 32
// values along K, which the matrix core consumes directly:
// v_mfma_scale_f32_16x16x128_f8f6f4 with both operands in FP4 multiplies a
// 16 x 128 block by a 128 x 16 block, applies each lane's E8M0 scale to the 32
// values it supplies, and accumulates in fp32. There is no unpacking and no
// per-group rescale on the vector ALU.
//
// Operand layout of the instruction (checked on the device): lane l supplies
// row (or column) l%16 and K values 32*(l/16) .. +31 of the 128, as 16 bytes of
// packed codes, plus one E8M0 byte for that 32-block, chosen from a 32-bit
// register by the op_sel immediate. The weight fragment is the first operand,
// so a lane ends up with 4 consecutive columns of one row of each 16 x 16
// output block, as in the INT4 kernel, and the same epilogue pieces
// (k2_common.hpp) finish the tile: the low-rank up-projection seeds the
// accumulators before the K loop (from the pre-kernel's fp16 D in operand
// order: one 16-byte load per row block and 32 ranks, nothing converted), the
// bias and the stores follow it (a full quarter of an fp16 Y goes through the
// then idle operand LDS and out in whole cache lines).
//
// Data movement. One instruction takes 16 cycles on a SIMD and consumes 2 KB
// of operands, so operand delivery, not arithmetic, bounds this kernel. Both
// operands arrive in the tiled layouts of svdq.h: the 16 bytes every lane needs
// for one 16-row block and one chunk of 128 form one contiguous 1 KB run, and
// the exponent bytes for four such blocks one contiguous 256-byte run (a
// 32-bit word per lane whose byte i belongs to block i).
// - Full tiles copy every block of a chunk from global memory into LDS once
//   per workgroup, with direct-to-LDS loads (global_load_lds: no registers),
//   and each wave reads its blocks from LDS. Loading them per wave instead
//   fetched each block twice (two waves share every row and column panel)
//   and kept the vector memory address unit 72% busy. Three LDS stages: while
//   chunk c's matrix instructions run, chunk c+1 is read into registers and
//   chunk c+2 is copied into the stage chunk c-1 left; one barrier per chunk.
//   The waits are written out (s_waitcnt with the count of one chunk's copies,
//   then s_barrier) because the compiler's own would wait for every copy.
// - Quarter tiles (a thin last round) load straight into registers, one
//   coalesced 1 KB load per block and chunk; the K loop keeps NS chunks in
//   flight and has no branch, so the wait counter only ever waits for the
//   oldest chunk; chunk numbers past the end are clamped to the last chunk
//   (repeated loads, never used).
//
// Tiling: a 256-thread workgroup computes a 2*WTM x 2*WTN tile, each wave a
// WTM x WTN quarter: 256 x 128 tiles of 128 x 64 waves (128 fp32 accumulators
// per lane), and for a thin last round 128 x 64 tiles of 64 x 32 waves.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.hpp"
#include "device_launch.hpp"
#include "k2_common.hpp"

namespace svdq {

namespace {

constexpr int NT = 256;             // threads per workgroup
constexpr int kChunk = 128;         // K values per matrix instruction
constexpr int kCodeBlock = 1024;    // tiled codes per 16 rows and chunk
constexpr int kExpBlock = 256;      // tiled exponents per 64 rows and chunk
constexpr int NS = 2;               // chunks in flight per wave

typedef int v8i __attribute__((ext_vector_type(8)));

template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Operands of one chunk for one wave: NBM activation and NBN weight blocks,
// and their exponent words (one per 64 rows).
template <int NBM, int NBN>
struct MxFrags {
  static constexpr int SM = (NBM + 3) / 4, SN = (NBN + 3) / 4;
  uint4 A[NBM], B[NBN];
  uint32_t sa[SM], sb[SN];
};

__device__ __forceinline__ v8i as_operand(uint4 v) {
  return v8i{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z),
             static_cast<int>(v.w), 0, 0, 0, 0};
}

// acc[I][J] += (weight block J) x (activation block I) over one chunk
template <int NBM, int NBN, int I = 0, int J = 0>
__device__ __forceinline__ void mfma_chunk(v4f (&acc)[NBM][NBN], const MxFrags<NBM, NBN>& f) {
  if constexpr (I < NBM) {
    if constexpr (J < NBN) {
      acc[I][J] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          as_operand(f.B[J]), as_operand(f.A[I]), acc[I][J], 4, 4, J % 4,
          static_cast<int>(f.sb[J / 4]), I % 4, static_cast<int>(f.sa[I / 4]));
      mfma_chunk<NBM, NBN, I, J + 1>(acc, f);
    } else {
      mfma_chunk<NBM, NBN, I + 1, 0>(acc, f);
    }
  }
}

// One tile of Y: rows m0 .. m0 + 2*WTM - 1, columns n0 .. n0 + 2*WTN - 1.
// m0 is a multiple of 2*WTM and n0 of 2*WTN.
template <int WTM, int WTN, bool Y_F16, bool GELU>
__device__ __forceinline__ void mx_tile(
    const uint8_t* __restrict__ a_codes_t, const uint8_t* __restrict__ a_exps_t,
    const uint8_t* __restrict__ w_codes_t, const uint8_t* __restrict__ w_exps_t,
    const uint16_t* __restrict__ Dt, const uint16_t* __restrict__ L2t, int R,
    const float* __restrict__ bias, void* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int64_t m0, int64_t n0) {
  constexpr int NBM = WTM / 16, NBN = WTN / 16;
  using Frags = MxFrags<NBM, NBN>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t C = (K + kChunk - 1) / kChunk;
  const int64_t ms = m0 + wm * WTM, ns = n0 + wn * WTN;   // the wave's first row and column
  const int64_t mb_last = (M + 15) / 16 - 1, nb_last = (N + 15) / 16 - 1;
  const int64_t mg_last = (M + 63) / 64 - 1, ng_last = (N + 63) / 64 - 1;

  // Block bases, the same for the whole wave; blocks past the last row are
  // clamped to it (their results are never stored).
  const uint8_t* ab[NBM];
  const uint8_t* bb[NBN];
  const uint8_t* ae[Frags::SM];
  const uint8_t* be[Frags::SN];
#pragma unroll
  for (int i = 0; i < NBM; ++i) {
    const int64_t b = ms / 16 + i;
    ab[i] = a_codes_t + (b < mb_last ? b : mb_last) * C * kCodeBlock;
  }
#pragma unroll
  for (int j = 0; j < NBN; ++j) {
    const int64_t b = ns / 16 + j;
    bb[j] = w_codes_t + (b < nb_last ? b : nb_last) * C * kCodeBlock;
  }
#pragma unroll
  for (int s = 0; s < Frags::SM; ++s) {
    const int64_t g = ms / 64 + s;
    ae[s] = a_exps_t + (g < mg_last ? g : mg_last) * C * kExpBlock;
  }
#pragma unroll
  for (int s = 0; s < Frags::SN; ++s) {
    const int64_t g = ns / 64 + s;
    be[s] = w_exps_t + (g < ng_last ? g : ng_last) * C * kExpBlock;
  }
  // a wave that starts 16*k rows into a 64-row group (only 32-row waves do)
  // finds its blocks' exponents from byte k on
  const int sha = WTM < 64 ? 8 * static_cast<int>((ms % 64) / 16) : 0;
  const int shb = WTN < 64 ? 8 * static_cast<int>((ns % 64) / 16) : 0;

  auto load = [&](Frags& f, int64_t c) {
    c = c < C ? c : C - 1;
    const int64_t co = c * kCodeBlock + 16 * lane, eo = c * kExpBlock + 4 * lane;
#pragma unroll
    for (int i = 0; i < NBM; ++i) f.A[i] = *reinterpret_cast<const uint4*>(ab[i] + co);
#pragma unroll
    for (int j = 0; j < NBN; ++j) f.B[j] = *reinterpret_cast<const uint4*>(bb[j] + co);
#pragma unroll
    for (int s = 0; s < Frags::SM; ++s) f.sa[s] = *reinterpret_cast<const uint32_t*>(ae[s] + eo);
#pragma unroll
    for (int s = 0; s < Frags::SN; ++s) f.sb[s] = *reinterpret_cast<const uint32_t*>(be[s] + eo);
  };
  auto align_exps = [&](Frags& f) {
    if constexpr (WTM < 64) f.sa[0] >>= sha;
    if constexpr (WTN < 64) f.sb[0] >>= shb;
  };

  // The first chunk's loads go out first; the low-rank up-projection then
  // starts the accumulators (acc = fp16(D) . L2) while they are in flight,
  // instead of exposing its own loads after the K loop; the second chunk's
  // loads follow (issuing them earlier would hold more registers than there
  // are next to the branch's operands).
  static_assert(NS == 2, "the prologue below is written for two chunks in flight");
  Frags f[NS];
  load(f[0], 0);

  v4f acc[NBM][NBN];
#pragma unroll
  for (int i = 0; i < NBM; ++i)
#pragma unroll
    for (int j = 0; j < NBN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  lowrank_up_dt<WTM, WTN>(acc, Dt, L2t, R, M, N, m0, n0);
  load(f[1], 1);
  int64_t c0 = 0;
  for (; c0 + NS <= C; c0 += NS) {
    static_for<NS>([&](auto S) {
      align_exps(f[S.value]);
      mfma_chunk<NBM, NBN>(acc, f[S.value]);
      // keep each chunk's loads together and behind its matrix instructions,
      // so that the loads in flight are always the newest ones
      __builtin_amdgcn_sched_barrier(0);
      load(f[S.value], c0 + S.value + NS);
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  static_for<NS>([&](auto S) {
    if (c0 + S.value < C) {
      align_exps(f[S.value]);
      mfma_chunk<NBM, NBN>(acc, f[S.value]);
    }
  });

  bias_store<WTM, WTN, Y_F16, GELU>(acc, bias, Y, M, N, ldy, m0, n0);
}

// Full 256 x 128 tile with the operands shared through LDS (see the top of
// the file): each wave copies 4 activation blocks, 2 weight blocks and one
// exponent block of each (waves 2 and 3 copy the weight exponents again,
// which keeps every wave's copy count at 8), and reads its 8 activation and 4
// weight blocks and their exponent words.
struct alignas(16) MxStage {
  uint8_t a[16][kCodeBlock];        // activation blocks of the tile's 256 rows
  uint8_t b[8][kCodeBlock];         // weight blocks of its 128 columns
  uint8_t ea[4][kExpBlock];         // activation exponent blocks (64 rows each)
  uint8_t eb[2][kExpBlock];         // weight exponent blocks
};

#define LDSP(p) ((__attribute__((address_space(3))) void*)(p))

template <bool Y_F16, bool GELU>
__device__ __forceinline__ void mx_tile_lds(
    MxStage (&st)[3], const uint8_t* __restrict__ a_codes_t, const uint8_t* __restrict__ a_exps_t,
    const uint8_t* __restrict__ w_codes_t, const uint8_t* __restrict__ w_exps_t,
    const uint16_t* __restrict__ Dt, const uint16_t* __restrict__ L2t, int R,
    const float* __restrict__ bias, void* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int64_t m0, int64_t n0) {
  constexpr int WTM = 128, WTN = 64, NBM = 8, NBN = 4;
  using Frags = MxFrags<NBM, NBN>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t C = (K + kChunk - 1) / kChunk;
  const int64_t mb_last = (M + 15) / 16 - 1, nb_last = (N + 15) / 16 - 1;
  const int64_t mg_last = (M + 63) / 64 - 1, ng_last = (N + 63) / 64 - 1;
  // this wave's share of the copies: activation blocks 4w .. 4w+3, weight
  // blocks 2w, 2w+1, activation exponent block w and weight exponent block
  // w % 2 (waves 2 and 3 copy the same bytes as 0 and 1)
  const uint8_t* ga[4];
  const uint8_t* gb[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t b = m0 / 16 + 4 * wave + i;
    ga[i] = a_codes_t + (b < mb_last ? b : mb_last) * C * kCodeBlock + 16 * lane;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t b = n0 / 16 + 2 * wave + j;
    gb[j] = w_codes_t + (b < nb_last ? b : nb_last) * C * kCodeBlock + 16 * lane;
  }
  const int64_t gea_b = m0 / 64 + wave, geb_b = n0 / 64 + (wave & 1);
  const uint8_t* gea = a_exps_t + (gea_b < mg_last ? gea_b : mg_last) * C * kExpBlock + 4 * lane;
  const uint8_t* geb = w_exps_t + (geb_b < ng_last ? geb_b : ng_last) * C * kExpBlock + 4 * lane;

  auto copy = [&](MxStage& s, int64_t c) {
    c = c < C ? c : C - 1;
    const int64_t co = c * kCodeBlock, eo = c * kExpBlock;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(ga[i] + co, LDSP(&s.a[4 * wave + i][0]), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_global_load_lds(gb[j] + co, LDSP(&s.b[2 * wave + j][0]), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(gea + eo, LDSP(&s.ea[wave][0]), 4, 0, 0);
    __builtin_amdgcn_global_load_lds(geb + eo, LDSP(&s.eb[wave & 1][0]), 4, 0, 0);
  };
  auto read = [&](Frags& f, const MxStage& s) {
#pragma unroll
    for (int i = 0; i < NBM; ++i) f.A[i] = *reinterpret_cast<const uint4*>(&s.a[NBM * wm + i][16 * lane]);
#pragma unroll
    for (int j = 0; j < NBN; ++j) f.B[j] = *reinterpret_cast<const uint4*>(&s.b[NBN * wn + j][16 * lane]);
#pragma unroll
    for (int t = 0; t < 2; ++t) f.sa[t] = *reinterpret_cast<const uint32_t*>(&s.ea[2 * wm + t][4 * lane]);
    f.sb[0] = *reinterpret_cast<const uint32_t*>(&s.eb[wn][4 * lane]);
  };
  // all of this wave's copies and LDS reads done, then every wave's
  constexpr int kWaitAll = 0x0070;   // vmcnt(0) expcnt(7) lgkmcnt(0)
  auto sync = [&]() {
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_s_barrier();
  };

  copy(st[0], 0);
  copy(st[1], 1);
  v4f acc[NBM][NBN];
#pragma unroll
  for (int i = 0; i < NBM; ++i)
#pragma unroll
    for (int j = 0; j < NBN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  lowrank_up_dt<WTM, WTN>(acc, Dt, L2t, R, M, N, m0, n0);
  sync();                            // chunks 0 and 1 in stages 0 and 1
  Frags f[2];
  read(f[0], st[0]);
  // iteration c: chunk c's operands are in f[c % 2]; chunk c+1 is in stage
  // (c+1) % 3; chunk c+2 is copied into stage (c+2) % 3, which held chunk
  // c-1 (read two iterations ago, before the last barrier)
  constexpr int kWaitCopies = 0x0078;  // vmcnt(8) expcnt(7) lgkmcnt(0): one chunk's copies may fly
  int64_t c = 0;
  int s1 = 1, s2 = 2;                // stages of chunks c+1 and c+2
  for (; c + 2 <= C; c += 2) {
    static_for<2>([&](auto S) {
      constexpr int P = S.value;
      copy(st[s2], c + P + 2);
      __builtin_amdgcn_s_waitcnt(kWaitCopies);
      __builtin_amdgcn_s_barrier();  // chunk c+P+1 copied by all waves
      read(f[P ^ 1], st[s1]);
      __builtin_amdgcn_sched_barrier(0);
      mfma_chunk<NBM, NBN>(acc, f[P]);
      __builtin_amdgcn_sched_barrier(0);
      s1 = s2;
      s2 = s2 == 2 ? 0 : s2 + 1;
    });
  }
  if (c < C) mfma_chunk<NBM, NBN>(acc, f[0]);
  // the copies of chunks past the end land in LDS no later wave reads; wait
  // for them before the workgroup's LDS can be handed on
  sync();
  static_assert(sizeof(MxStage) * 3 >= 4 * WTM * 128, "each wave stages a WTM x 64 fp16 tile");
  if (Y_F16 && lds_store_ok<WTM, WTN>(Y, ldy, M, N, m0, n0))
    bias_store_lds_f16<WTM, WTN, GELU>(acc, bias, static_cast<_Float16*>(Y), ldy, m0, n0,
                                       reinterpret_cast<uint8_t*>(&st[0]) + wave * WTM * 128);
  else
    bias_store<WTM, WTN, Y_F16, GELU>(acc, bias, Y, M, N, ldy, m0, n0);
}

constexpr int kFullM = 256, kFullN = 128;     // full tile; quarters are 128 x 64

// Workgroups 0 .. n_full-1 take the first n_full full tiles of the banded
// order; the remaining workgroups take the leftover tiles in quarters.
template <bool Y_F16, bool GELU>
__global__ __launch_bounds__(NT, 2) void k2_mx_kernel(
    const uint8_t* __restrict__ a_codes_t, const uint8_t* __restrict__ a_exps_t,
    const uint8_t* __restrict__ w_codes_t, const uint8_t* __restrict__ w_exps_t,
    const uint16_t* __restrict__ Dt, const uint16_t* __restrict__ L2t, int R,
    const float* __restrict__ bias, void* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int tiles_m, int tiles_n, int n_full) {
  __shared__ MxStage st[3];
  const int b = static_cast<int>(blockIdx.x);
  int tm, tn;
  if (b < n_full) {
    banded_tile(xcd_contiguous(b, n_full), tiles_m, tiles_n, tm, tn);
    mx_tile_lds<Y_F16, GELU>(st, a_codes_t, a_exps_t, w_codes_t, w_exps_t, Dt, L2t,
                             R, bias, Y, M, N, K, ldy,
                             static_cast<int64_t>(tm) * kFullM,
                             static_cast<int64_t>(tn) * kFullN);
  } else {
    const int qb = b - n_full;
    const int quarter = qb & 3;
    banded_tile(n_full + (qb >> 2), tiles_m, tiles_n, tm, tn);
    mx_tile<kFullM / 4, kFullN / 4, Y_F16, GELU>(
        a_codes_t, a_exps_t, w_codes_t, w_exps_t, Dt, L2t, R, bias, Y, M, N, K, ldy,
        static_cast<int64_t>(tm) * kFullM + (kFullM / 2) * (quarter >> 1),
        static_cast<int64_t>(tn) * kFullN + (kFullN / 2) * (quarter & 1));
  }
}

}  // namespace

hipError_t launch_k2_mx(const uint8_t* a_codes_t, const uint8_t* a_exps_t,
                        const uint8_t* w_codes_t, const uint8_t* w_exps_t, const uint16_t* Dt,
                        const uint16_t* L2t, int R, const float* bias, void* Y, bool y_f16,
                        int64_t M, int64_t N, int64_t K, int64_t ldy, bool gelu,
                        hipStream_t stream) {
  const int tiles_m = static_cast<int>((M + kFullM - 1) / kFullM);
  const int tiles_n = static_cast<int>((N + kFullN - 1) / kFullN);
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
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, a_codes_t, a_exps_t, w_codes_t, w_exps_t,
                       Dt, L2t, R, bias, Y, M, N, K, ldy, tiles_m, tiles_n, n_full);
  };
  if (y_f16)
    gelu ? go(k2_mx_kernel<true, true>) : go(k2_mx_kernel<true, false>);
  else
    gelu ? go(k2_mx_kernel<false, true>) : go(k2_mx_kernel<false, false>);
  return hipGetLastError();
}

}  // namespace svdq
