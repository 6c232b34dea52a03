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
// per-group rescale on the vector ALU, so unlike the INT4 kernel this one is
// bound by the matrix core and by operand traffic, not by vector arithmetic.
//
// Operand layout of the instruction (checked on the device): lane l supplies
// row (or column) l%16 and K values 32*(l/16) .. +31 of the 128, as 16 bytes of
// packed codes (element 2j in the low nibble, the canonical layout), plus one
// E8M0 byte for that 32-block, chosen from a 32-bit register by the op_sel
// immediate. The weight fragment is the first operand, so a lane ends up with
// 4 consecutive columns of one row of each 16 x 16 output block, as in the
// INT4 kernel, and the same epilogue (k2_common.hpp) finishes the tile.
//
// Tiling: a 256-thread workgroup computes a 2*WT x 2*WT tile, each wave a
// WT x WT quarter. The K loop runs over chunks of 128 (64 bytes of codes per
// row) through double-buffered LDS:
//   operands  sm.a/b[buf][row block][slot]: the 16 bytes lane l reads for a
//             row block sit in one slot, so every operand is one 16-byte LDS
//             read; slot = 16*kq + (r ^ 4*kq) for row r%16 and 16-byte piece
//             kq, which keeps both the loader's stores (4 rows x 4 pieces per
//             16 lanes) and the readers' loads (16 rows of one piece) on
//             distinct banks;
//   scales    sm.sa/sb[buf][half][lane]: the 4 E8M0 bytes (row blocks i = 0..3
//             of the wave's half) that lane l needs, one 32-bit LDS read; the
//             matrix instruction picks byte i with op_sel.
// A K that is an odd multiple of 64 ends with a half chunk: its missing half
// is zero codes with scale byte 127 (2^0), which adds exactly zero.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "device_launch.hpp"
#include "k2_common.hpp"

namespace svdq {

namespace {

constexpr int NT = 256;             // threads per workgroup
constexpr int kChunk = 128;         // K values per matrix instruction
constexpr int kChunkBytes = 64;     // packed codes per row and chunk
constexpr int kMxBlock = 32;        // values per E8M0 scale

typedef int v8i __attribute__((ext_vector_type(8)));

template <int WT>
struct MxSmem {
  uint4 a[2][2 * WT / 16][64];      // activation operands [buf][row block][slot]
  uint4 b[2][2 * WT / 16][64];      // weight operands
  uint32_t sa[2][2][64];            // activation scales [buf][wm][lane], byte i = row block i
  uint32_t sb[2][2][64];            // weight scales [buf][wn][lane], byte j = column block j
};

__device__ __forceinline__ int slot_of(int kq, int r) { return 16 * kq + (r ^ (kq << 2)); }

// One chunk of the tile, between its global load and its LDS store.
//   codes: thread t loads piece kq = t%4 of tile rows t/4 (+64 for BT = 128),
//          of A and of B: each group of 4 threads reads one row's 64 bytes.
//   scales: threads 0 .. BT-1 load the 4 E8M0 bytes of A row t, threads
//          BT .. 2BT-1 those of B row t-BT (two 16-bit loads: a row's
//          exponents are only 2-byte aligned when K % 128 == 64).
// Rows past M or N are clamped to the last one (their results are never
// stored), so every load is in bounds.
template <int WT>
struct MxLoader {
  static constexpr int BT = 2 * WT;
  static constexpr int NR = BT / 64;                  // code rows per thread and operand
  const uint8_t* arow[NR];
  const uint8_t* brow[NR];
  const uint16_t* srow;
  uint4 ca[NR], cb[NR];
  uint32_t sc;
  bool has_scale;

  __device__ __forceinline__ void init(const uint8_t* a_codes, const uint8_t* a_e8m0,
                                       const uint8_t* w_codes, const uint8_t* w_e8m0,
                                       int64_t m0, int64_t n0, int64_t M, int64_t N, int64_t K) {
    const int t = threadIdx.x;
    const int64_t kb = K / 2, ks = K / kMxBlock;
    auto clamp_m = [&](int64_t r) { return m0 + r < M ? m0 + r : M - 1; };
    auto clamp_n = [&](int64_t r) { return n0 + r < N ? n0 + r : N - 1; };
    const int kq = t & 3;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = (t >> 2) + 64 * i;
      arow[i] = a_codes + clamp_m(r) * kb + 16 * kq;
      brow[i] = w_codes + clamp_n(r) * kb + 16 * kq;
    }
    has_scale = t < 2 * BT;
    const int s = has_scale ? t : 0;
    srow = reinterpret_cast<const uint16_t*>(s < BT ? a_e8m0 + clamp_m(s) * ks
                                                    : w_e8m0 + clamp_n(s - BT) * ks);
  }

  // chunk c; `full`: all 128 K values exist (else only the first 64)
  __device__ __forceinline__ void load(int64_t c, bool full) {
    const int kq = threadIdx.x & 3;
    const bool live = full || kq < 2;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      ca[i] = live ? *reinterpret_cast<const uint4*>(arow[i] + c * kChunkBytes) : make_uint4(0, 0, 0, 0);
      cb[i] = live ? *reinterpret_cast<const uint4*>(brow[i] + c * kChunkBytes) : make_uint4(0, 0, 0, 0);
    }
    const uint32_t lo = srow[2 * c];
    const uint32_t hi = full ? srow[2 * c + 1] : 0x7F7Fu;
    sc = lo | (hi << 16);
  }

  __device__ __forceinline__ void store(MxSmem<WT>& sm, int buf) const {
    const int t = threadIdx.x;
    const int kq = t & 3;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = (t >> 2) + 64 * i;
      sm.a[buf][r >> 4][slot_of(kq, r & 15)] = ca[i];
      sm.b[buf][r >> 4][slot_of(kq, r & 15)] = cb[i];
    }
    if (has_scale) {
      const bool is_b = t >= BT;
      const int r = is_b ? t - BT : t;                 // tile row (A) or column (B)
      const int half = r / WT, blk = (r % WT) >> 4, rr = r & 15;
      uint8_t* dst = reinterpret_cast<uint8_t*>(is_b ? sm.sb[buf][half] : sm.sa[buf][half]);
#pragma unroll
      for (int kq2 = 0; kq2 < 4; ++kq2) dst[4 * (16 * kq2 + rr) + blk] = (sc >> (8 * kq2)) & 0xFFu;
    }
  }
};

template <int NB>
struct MxFrags {
  uint4 A[NB], B[NB];
  uint32_t sa, sb;
};

template <int WT>
__device__ __forceinline__ void read_chunk(MxFrags<WT / 16>& f, const MxSmem<WT>& sm, int buf,
                                           int wm, int wn, int lane) {
  constexpr int NB = WT / 16;
  const int sl = slot_of(lane >> 4, lane & 15);
#pragma unroll
  for (int i = 0; i < NB; ++i) f.A[i] = sm.a[buf][wm * NB + i][sl];
#pragma unroll
  for (int j = 0; j < NB; ++j) f.B[j] = sm.b[buf][wn * NB + j][sl];
  f.sa = sm.sa[buf][wm][lane];
  f.sb = sm.sb[buf][wn][lane];
}

__device__ __forceinline__ v8i as_operand(uint4 v) {
  return v8i{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z),
             static_cast<int>(v.w), 0, 0, 0, 0};
}

// acc += (weight block j) x (activation block i) over one chunk; the scale
// bytes are byte j of sb and byte i of sa
template <int I, int J>
__device__ __forceinline__ v4f mfma_mx(const v4f& acc, const uint4& b, const uint4& a, uint32_t sb,
                                       uint32_t sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(as_operand(b), as_operand(a), acc, 4, 4,
                                                          J, static_cast<int>(sb), I,
                                                          static_cast<int>(sa));
}

template <int NB, int I = 0, int J = 0>
__device__ __forceinline__ void mfma_chunk(v4f (&acc)[NB][NB], const MxFrags<NB>& f) {
  if constexpr (I < NB) {
    if constexpr (J < NB) {
      acc[I][J] = mfma_mx<I, J>(acc[I][J], f.B[J], f.A[I], f.sb, f.sa);
      mfma_chunk<NB, I, J + 1>(acc, f);
    } else {
      mfma_chunk<NB, I + 1, 0>(acc, f);
    }
  }
}

template <int WT, bool Y_F16, bool GELU>
__device__ __forceinline__ void mx_tile(
    MxSmem<WT>& sm, const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_e8m0,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_e8m0,
    const float* __restrict__ D, const uint16_t* __restrict__ L2t, int R,
    const float* __restrict__ bias, void* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int64_t m0, int64_t n0) {
  constexpr int NB = WT / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t C = (K + kChunk - 1) / kChunk;        // chunks; the last may be half
  const bool last_full = (K % kChunk) == 0;
  auto full = [&](int64_t c) { return c + 1 < C || last_full; };

  v4f acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Pipeline: LDS holds chunks c and c+1, registers hold chunk c+2 between
  // its global load and its store, and the operands of chunk c+1 are read
  // from LDS while the matrix instructions of chunk c run.
  MxLoader<WT> ld;
  ld.init(a_codes, a_e8m0, w_codes, w_e8m0, m0, n0, M, N, K);
  ld.load(0, full(0));
  ld.store(sm, 0);
  if (C > 1) {
    ld.load(1, full(1));
    ld.store(sm, 1);
  }
  if (C > 2) ld.load(2, full(2));
  __syncthreads();

  MxFrags<NB> f;
  read_chunk<WT>(f, sm, 0, wm, wn, lane);
  for (int64_t c = 0; c < C; ++c) {
    mfma_chunk<NB>(acc, f);
    if (c + 1 < C) {
      const int buf = static_cast<int>(c & 1);
      __syncthreads();               // every wave has read chunk c; chunk c+1 is in LDS
      if (c + 2 < C) {
        ld.store(sm, buf);           // chunk c+2 replaces chunk c
        if (c + 3 < C) ld.load(c + 3, full(c + 3));
      }
      read_chunk<WT>(f, sm, buf ^ 1, wm, wn, lane);
    }
  }

  lowrank_bias_store<WT, Y_F16, GELU>(acc, D, L2t, R, bias, Y, M, N, ldy, m0, n0);
}

// Workgroups 0 .. n_full-1 take the first n_full 128 x 128 tiles of the banded
// order; the remaining workgroups take the leftover tiles in quarters.
template <bool Y_F16, bool GELU>
__global__ __launch_bounds__(NT, 2) void k2_mx_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_e8m0,
    const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_e8m0,
    const float* __restrict__ D, const uint16_t* __restrict__ L2t, int R,
    const float* __restrict__ bias, void* __restrict__ Y, int64_t M, int64_t N, int64_t K,
    int64_t ldy, int tiles_m, int tiles_n, int n_full) {
  __shared__ union {
    MxSmem<64> full;
    MxSmem<32> quarter;
  } sm;
  const int b = static_cast<int>(blockIdx.x);
  int tm, tn;
  if (b < n_full) {
    banded_tile(xcd_contiguous(b, n_full), tiles_m, tiles_n, tm, tn);
    mx_tile<64, Y_F16, GELU>(sm.full, a_codes, a_e8m0, w_codes, w_e8m0, D, L2t, R, bias, Y, M, N,
                             K, ldy, static_cast<int64_t>(tm) * 128,
                             static_cast<int64_t>(tn) * 128);
  } else {
    const int qb = b - n_full;
    const int quarter = qb & 3;
    banded_tile(n_full + (qb >> 2), tiles_m, tiles_n, tm, tn);
    mx_tile<32, Y_F16, GELU>(sm.quarter, a_codes, a_e8m0, w_codes, w_e8m0, D, L2t, R, bias, Y, M,
                             N, K, ldy, static_cast<int64_t>(tm) * 128 + 64 * (quarter >> 1),
                             static_cast<int64_t>(tn) * 128 + 64 * (quarter & 1));
  }
}

}  // namespace

hipError_t launch_k2_mx(const uint8_t* a_codes, const uint8_t* a_e8m0, const uint8_t* w_codes,
                        const uint8_t* w_e8m0, const float* D, const uint16_t* L2t, int R,
                        const float* bias, void* Y, bool y_f16, int64_t M, int64_t N, int64_t K,
                        int64_t ldy, bool gelu, hipStream_t stream) {
  const int tiles_m = static_cast<int>((M + 127) / 128);
  const int tiles_n = static_cast<int>((N + 127) / 128);
  const int T = tiles_m * tiles_n;
  const int S = resident_slots();
  const int left = T < S ? T : T % S;
  const int n_quarter_tiles = (left > 0 && 2 * left <= S) ? left : 0;
  const int n_full = T - n_quarter_tiles;
  const dim3 grid(static_cast<unsigned>(n_full + 4 * n_quarter_tiles)), block(NT);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, a_codes, a_e8m0, w_codes, w_e8m0, D, L2t,
                       R, bias, Y, M, N, K, ldy, tiles_m, tiles_n, n_full);
  };
  if (y_f16)
    gelu ? go(k2_mx_kernel<true, true>) : go(k2_mx_kernel<true, false>);
  else
    gelu ? go(k2_mx_kernel<false, true>) : go(k2_mx_kernel<false, false>);
  return hipGetLastError();
}

}  // namespace svdq
