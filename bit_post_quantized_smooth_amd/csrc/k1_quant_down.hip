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
// The MXFP4 instance (MX = true) replaces the quantizer step: per row and
// block of 32 channels, the E8M0 exponent of the block's absmax and E2M1
// codes (OCP Microscaling v1.0, the CDNA4 counterpart of the 4-bit float
// version on the taicenter.com news page, hardware co-design section), and
// the codes and exponents go out in the tiled layouts K2-MX reads (svdq.h);
// the rest of the kernel is the same.
//
// Work split: a workgroup owns 16 rows; its waves (8, or 4 at high rank) take
// the 64-channel groups round-robin.
//
// Lane map per wave and group: lane l holds row l%16 and channels
// 16*(l/16) .. +15, which is exactly what v_mfma_f32_16x16x32_f16 wants for
// its two K-halves (8 consecutive channels per operand), so the fp16 values
// of the down-projection never leave the registers. A row's group is spread
// over the lanes r, r+16, r+32, r+48: its absmax is a reduction over those
// four lanes with the gfx950 lane-swap instructions (v_permlane16_swap,
// v_permlane32_swap), and the four lanes write its 32 bytes of codes side by
// side. Each lane loads one smoothing factor per group (lane l: channel l of
// the group, one coalesced 256-byte load per wave) and takes the 16 it needs
// from the lanes of its 16-lane row with DPP row broadcasts. L1 arrives packed
// in the matrix instruction's operand order (see
// svdq_pack_lowrank_down), so each operand is one contiguous 1 KB load per
// wave. The per-wave partial D tiles are summed in LDS in a fixed order.
//
// Latency hiding: each wave keeps a ring of NB groups in registers; group i is
// processed while groups i+1 .. i+NB-1 are in flight, and its slot is then
// refilled with group i+NB. Every load is unconditional (rows past M, groups
// past the wave's last and column blocks past R/16 are clamped to valid
// addresses and their results discarded), so the compiler counts outstanding
// loads exactly and never waits for more than the one group it needs.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "device_launch.hpp"
#include "k2_common.hpp"

namespace svdq {

namespace {

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

// xh[i] = fp32(x[i]) * inv[i], rounded once to fp32. For fp16 X this is one
// v_fma_mix_f32 per value: fma(fp32(x), inv, -0) equals the product exactly
// (adding -0 changes no value, not even a zero's sign); `nz` is -0 in a
// register the compiler cannot see through, which keeps it from rewriting the
// fma as a conversion plus a multiply.
__device__ __forceinline__ void smooth16(const Raw<_Float16>& r, const float4* inv, float* xh,
                                         float nz) {
  const uint32_t w[8] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w,
                         r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
  const float iv[16] = {inv[0].x, inv[0].y, inv[0].z, inv[0].w, inv[1].x, inv[1].y,
                        inv[1].z, inv[1].w, inv[2].x, inv[2].y, inv[2].z, inv[2].w,
                        inv[3].x, inv[3].y, inv[3].z, inv[3].w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    xh[2 * i] = __builtin_fmaf(h2f(static_cast<uint16_t>(w[i] & 0xFFFFu)), iv[2 * i], nz);
    xh[2 * i + 1] = __builtin_fmaf(h2f(static_cast<uint16_t>(w[i] >> 16)), iv[2 * i + 1], nz);
  }
}

__device__ __forceinline__ void smooth16(const Raw<float>& r, const float4* inv, float* xh,
                                         float) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xh[4 * i] = r.v[i].x * inv[i].x;
    xh[4 * i + 1] = r.v[i].y * inv[i].y;
    xh[4 * i + 2] = r.v[i].z * inv[i].z;
    xh[4 * i + 3] = r.v[i].w * inv[i].w;
  }
}

// Lane J of each 16-lane row, in every lane of that row (DPP row_newbcast).
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + J,
                                                            0xF, 0xF, false));
}

// The 16 smoothing factors of a lane's channels 16q .. 16q+15, from one value
// per lane (lane 16q + j holds channel 16q + j's).
__device__ __forceinline__ void expand_inv(float v, float4 inv[4]) {
  inv[0] = make_float4(row_bcast<0>(v), row_bcast<1>(v), row_bcast<2>(v), row_bcast<3>(v));
  inv[1] = make_float4(row_bcast<4>(v), row_bcast<5>(v), row_bcast<6>(v), row_bcast<7>(v));
  inv[2] = make_float4(row_bcast<8>(v), row_bcast<9>(v), row_bcast<10>(v), row_bcast<11>(v));
  inv[3] = make_float4(row_bcast<12>(v), row_bcast<13>(v), row_bcast<14>(v), row_bcast<15>(v));
}

// Maxima of non-negative floats across lanes, on their bit patterns (for
// values >= 0 the unsigned order of the bits is the order of the values, and
// no NaN quieting is involved). permlane16_swap(v, v) hands every lane the
// value of lane l^16 in one of its two results, permlane32_swap(v, v) that of
// lane l^32.
__device__ __forceinline__ float max_xor16(float a) {
  const uint32_t b = __builtin_bit_cast(uint32_t, a);
  const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return __builtin_bit_cast(float, r[0] > r[1] ? r[0] : r[1]);
}
__device__ __forceinline__ float max_xor32(float a) {
  const uint32_t b = __builtin_bit_cast(uint32_t, a);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __builtin_bit_cast(float, r[0] > r[1] ? r[0] : r[1]);
}

// Codes of 8 values from the fp32 bit patterns of (value + 1.5 * 2^23), whose
// low byte is the value's two's-complement integer: byte j of the result is
// code 2j in its low nibble and code 2j+1 in its high nibble. Byte permutes
// gather the even and the odd codes, a bit-field insert merges them.
__device__ __forceinline__ uint32_t pack8_codes(const uint32_t* b) {
  constexpr uint32_t kLow2 = 0x0C0C0400u;        // [S1.byte0, S0.byte0, 0, 0]
  constexpr uint32_t kCat = 0x05040100u;         // [S1.byte0, S1.byte1, S0.byte0, S0.byte1]
  const uint32_t ev = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[6], b[4], kLow2),
                                            __builtin_amdgcn_perm(b[2], b[0], kLow2), kCat);
  const uint32_t od = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[5], kLow2),
                                            __builtin_amdgcn_perm(b[3], b[1], kLow2), kCat);
  return (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
}

constexpr float kInv7 = 0.142857149f;           // fp32(1/7) = 0x3E124925

// INT4 quantizer of one row's group of 64 (lanes r, r+16, r+32, r+48, 16
// values each): packed codes of this lane's 16 values and the group's fp16
// scale.
__device__ __forceinline__ void quantize_int4(const float* xh, uint32_t packed[2], uint16_t& s16) {
  // group absmax over this lane's 16 values, then across the 4 lanes of the row
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(xh[j]));
  a = max_xor32(max_xor16(a));
  // fp32(a / 7), correctly rounded, as one multiply by fp32(1/7) and one
  // FMA correction (division by a constant known in advance: Brisebarre,
  // Muller, Raina, IEEE Trans. Computers 2004); for the divisor 7 this is
  // exact for every non-negative finite fp32 a, which was checked
  // exhaustively against the IEEE division on the host.
  const float q7 = a * kInv7;
  const float s32 = fminf(__builtin_fmaf(__builtin_fmaf(-q7, 7.0f, a), kInv7, q7), 65504.0f);
  s16 = f2h(s32);
  const float sf = h2f(s16);
  // 1/s correctly rounded: the hardware reciprocal (within one ulp) and one
  // Newton step give exactly the IEEE quotient for every fp16 s (checked
  // exhaustively on the host, for any start within two floats of it)
  const float r0 = __builtin_amdgcn_rcpf(sf);
  const float rc = __builtin_fmaf(__builtin_fmaf(-sf, r0, 1.0f), r0, r0);
  const float inv = (sf == 0.f) ? 0.f : rc;
  // code = clamp(rint(xh * inv), -7, 7): clamping first gives the same
  // result, and adding 1.5 * 2^23 rounds half-to-even to an integer whose
  // low 4 bits are its two's-complement nibble.
  uint32_t bits[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float c = __builtin_amdgcn_fmed3f(xh[j] * inv, -7.f, 7.f);
    bits[j] = __builtin_bit_cast(uint32_t, c + kMagicF);
  }
  packed[0] = pack8_codes(bits);
  packed[1] = pack8_codes(bits + 8);
}

// MXFP4 quantizer of one row's two 32-channel blocks (lanes r, r+16 hold the
// first, lanes r+32, r+48 the second): packed E2M1 codes of this lane's 16
// values and the E8M0 byte of its block.
// The shared exponent is e = floor(log2 amax) - 2, at least -127, i.e. the
// E8M0 byte is amax's biased exponent field minus 2, floored at 0. Values are
// first multiplied by 2^-e (exact: a power of two, and every product that is
// not a normal fp32 is below 0.25 and gives a zero code of the same sign),
// then converted with scale 1 by v_cvt_scalef32_pk_fp4_f32, which rounds to
// the nearest E2M1 value, ties to even, and saturates at 6.
__device__ __forceinline__ void quantize_mx(const float* xh, uint32_t packed[2], uint32_t& e8out) {
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(xh[j]));
  a = max_xor16(a);
  const int ex = static_cast<int>(__builtin_bit_cast(uint32_t, a) >> 23);
  const int e8 = ex > 2 ? ex - 2 : 0;
  const float mult = __builtin_bit_cast(float, static_cast<uint32_t>(254 - e8) << 23);
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    uint32_t w = 0u;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xh[8 * d + 0] * mult, xh[8 * d + 1] * mult, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xh[8 * d + 2] * mult, xh[8 * d + 3] * mult, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xh[8 * d + 4] * mult, xh[8 * d + 5] * mult, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xh[8 * d + 6] * mult, xh[8 * d + 7] * mult, 1.0f, 3);
    packed[d] = w;
  }
  e8out = static_cast<uint32_t>(e8);
}

// L1 operands travel in the ring up to rank 128; above that they would not fit
// in registers next to the accumulators and are loaded just before use.
template <int NCB>
constexpr int ring_l1_blocks() { return NCB <= 8 ? NCB : 0; }

// Waves per workgroup: 8 while the LDS tiles of all waves fit next to a second
// resident workgroup, else 4.
template <int NCB>
constexpr int k1_waves() { return NCB <= 4 ? 8 : 4; }

// Everything one lane reads for one group: its 16 X values in each of the
// workgroup's RT row tiles, one smoothing factor (the lane's 16 come from its
// row's lanes) and, per column block of D, its two packed L1 operands (both
// shared by the row tiles).
template <typename XT, int NCB, int RT>
struct GroupIn {
  Raw<XT> x[RT];
  bool valid[RT];        // convolution: the tap lies inside the image (else the values are 0)
  float inv1;            // smoothing factor of channel 16*(lane/16) + lane%16 of the group
  v8h l1[ring_l1_blocks<NCB>() > 0 ? ring_l1_blocks<NCB>() : 1][2];
};

// a_codes, a_meta: INT4 codes (M x K/2) and fp16 group scales (M x K/64), or
// for MX the tiled E2M1 codes and E8M0 exponents (see svdq.h).
// RT: row tiles of 16 per workgroup. With RT = 2 every wave quantizes the same
// group of two row tiles with one set of smoothing factors and L1 operands,
// which halves their (cached) traffic per row; used when there are rows
// enough to keep every compute unit busy.
// CONV: X is an NHWC image and the rows are the patches of the convolution cg
// (the chattools.cn overview says the method applies to UNet backbones; the
// convolution is the linear layer on its patch matrix): row p is the output
// pixel (b, oh, ow), group g the 64 channels cb*64 .. +63 of tap (kh, kw) with
// g = (kh*KW + kw)*C/64 + cb. A lane reads its 16 channels at input pixel
// (oh*stride + kh - pad, ow*stride + kw - pad) or, outside the image, loads a
// clamped pixel and uses zeros, so every load stays unconditional.
// FMT: what the quantizer step writes (K1Fmt): the canonical INT4 codes and
// fp16 scales, the MXFP4 tiled codes and exponents, or the INT4 operands of
// the tiled GEMM (K2T): per 16-row block and group one 1 KB block in the
// matrix instruction's lane order (lane 16q + r: row r, codes 16q .. 16q+15
// of the group, widened to int8 16*q in widen_codes' order) and the scale in
// fp32, in the 128-row band layout of svdq.h.
// SPLIT: the instance that splits rows over S workgroups (S is 1 in the others,
// whose code then carries none of the slice arithmetic).
template <typename XT, int NCB, int NB, int FMT, bool CONV, int RT, int WV, bool SPLIT = false>
__global__ __launch_bounds__(64 * WV, WV >= 16 ? 1 : 2) void k1_quant_down_kernel(
    const XT* __restrict__ X, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ inv_smooth, const uint16_t* __restrict__ L1p, int R,
    uint8_t* __restrict__ a_codes, void* __restrict__ a_meta, float* __restrict__ D,
    ConvGeom cg, int S_arg, float* __restrict__ Dpart) {
#pragma clang fp contract(off)
  const int S = SPLIT ? S_arg : 1;
  constexpr bool MX = FMT == kK1Mx;
  constexpr bool TILED = FMT == kK1Int4Tiled;
  constexpr int WAVES = WV;
  constexpr int NCBA = NCB > 0 ? NCB : 1;
  __shared__ float dpart[WAVES][16 * RT][NCBA * 16];
  const int lane = threadIdx.x & 63;
  // the wave index is the same in all lanes: keep it (and everything derived
  // from it: group numbers, group offsets) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  // lane map: row qr = rl of each row tile, channels 16*c4 .. +15 of each group
  const int rl = lane & 15, q = lane >> 4;
  const int qr = rl, c4 = q;
  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin; renumber
  // so each XCD takes one contiguous run of row tiles (neighbouring output
  // pixels of a convolution read the same input rows, which then stay in
  // that XCD's L2)
  // With S slices, workgroup (tile, slice) takes the slice's run of groups
  // and leaves its partial D in Dpart for k1_reduce_kernel.
  const int unit = xcd_contiguous(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int tile = unit / S, slice = unit - tile * S;
  const int64_t row0 = static_cast<int64_t>(tile) * (16 * RT);
  const int G = static_cast<int>(K / kGroup);
  const int g_lo = static_cast<int>(static_cast<int64_t>(slice) * G / S);
  const int g_hi = static_cast<int>(static_cast<int64_t>(slice + 1) * G / S);
  const int ncb = R / 16;                            // real column blocks (<= NCB)
  // this wave's groups are g_lo + wave, g_lo + wave + WAVES, ...: n_mine of them
  const int n_mine = (g_hi - g_lo > wave) ? (g_hi - g_lo - wave + WAVES - 1) / WAVES : 0;
  const int64_t nchunks = (K + 127) / 128;

  // Per row tile: this lane's row (clamped to the last row for loads: rows
  // past M are computed and never stored, so every load is unconditional),
  // its X row, and where its codes and scales (or tiled codes and exponents) go
  const XT* xrow[RT];
  bool rvalid[RT];
  uint8_t* crow[RT];
  uint16_t* srow[RT];
  uint8_t* tcode[RT];
  uint8_t* texp[RT];
  int pix0[RT], ih0[RT], iw0[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t r0 = row0 + 16 * rt;
    const int64_t row = r0 + qr;
    rvalid[rt] = row < M;
    const int64_t rowc = rvalid[rt] ? row : M - 1;
    xrow[rt] = X + rowc * ldx + c4 * 16;
    crow[rt] = a_codes + row * (K / 2) + c4 * 8;
    srow[rt] = static_cast<uint16_t*>(a_meta) + row * G;
    // MXFP4: the tile's 1 KB code block per chunk of 128, and its 64-row
    // group's exponent blocks, in which its rows are byte (r0 % 64) / 16 of
    // each lane's dword
    tcode[rt] = a_codes + (r0 / 16) * nchunks * 1024;
    texp[rt] = static_cast<uint8_t*>(a_meta) + (r0 / 64) * nchunks * 256 + (r0 % 64) / 16;
    pix0[rt] = ih0[rt] = iw0[rt] = 0;
    if constexpr (CONV) {
      // convolution: this lane's output pixel (its first input pixel and the
      // pixel offset of its image)
      const int p = static_cast<int>(rowc);
      const int ohw = cg.OH * cg.OW;
      const int img = p / ohw, rem = p - img * ohw;
      const int oh = rem / cg.OW, ow = rem - oh * cg.OW;
      pix0[rt] = img * cg.H * cg.W;
      ih0[rt] = oh * cg.stride - cg.pad;
      iw0[rt] = ow * cg.stride - cg.pad;
    }
  }
  const v8h* l1b = reinterpret_cast<const v8h*>(L1p);

  // packed operand (g, c, h) of this lane
  auto l1_operand = [&](int g, int c, int h) -> const v8h* {
    const int cc = c < ncb ? c : ncb - 1;
    return l1b + static_cast<int64_t>((g * ncb + cc) * 2 + h) * 64 + lane;
  };

  auto load_group = [&](GroupIn<XT, NCB, RT>& in, int i) {
    int g = g_lo + wave + WAVES * i;
    g = g < g_hi ? g : g_hi - 1;
    const int k0 = g * kGroup;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if constexpr (CONV) {
        const int cbs = cg.C / kGroup;                  // channel groups per tap (uniform)
        const int t = g / cbs, cb = g - t * cbs;
        const int kh = t / cg.KW, kw = t - kh * cg.KW;
        const int ih = ih0[rt] + kh, iw = iw0[rt] + kw;
        in.valid[rt] = static_cast<unsigned>(ih) < static_cast<unsigned>(cg.H) &&
                       static_cast<unsigned>(iw) < static_cast<unsigned>(cg.W);
        const int ihc = ih < 0 ? 0 : (ih >= cg.H ? cg.H - 1 : ih);
        const int iwc = iw < 0 ? 0 : (iw >= cg.W ? cg.W - 1 : iw);
        const uint32_t off = static_cast<uint32_t>(pix0[rt] + ihc * cg.W + iwc) *
                                 static_cast<uint32_t>(cg.C) + cb * kGroup + c4 * 16;
        load_raw<XT>(in.x[rt], X + off);
      } else {
        in.valid[rt] = true;
        load_raw<XT>(in.x[rt], xrow[rt] + k0);
      }
    }
    in.inv1 = inv_smooth[k0 + lane];
    if constexpr (ring_l1_blocks<NCB>() > 0) {
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        in.l1[c][0] = *l1_operand(g, c, 0);
        in.l1[c][1] = *l1_operand(g, c, 1);
      }
    }
  };

  v4f acc[RT][NCBA];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int c = 0; c < NCBA; ++c) acc[rt][c] = v4f{0.f, 0.f, 0.f, 0.f};

  // -0 in a register the compiler cannot see through (see smooth16)
  float nz;
  __asm__("v_mov_b32 %0, 0x80000000" : "=v"(nz));

  GroupIn<XT, NCB, RT> ring[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) load_group(ring[b], b);

  for (int i0 = 0; i0 < n_mine; i0 += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = i0 + b;
      const int g = g_lo + wave + WAVES * i;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        uint32_t packed[2] = {0u, 0u};
        uint32_t meta = 0u;                  // fp16 scale, or the E8M0 byte
        if (i < n_mine) {
          float xh[16];
          float4 iv[4];
          expand_inv(ring[b].inv1, iv);
          smooth16(ring[b].x[rt], iv, xh, nz);
          if constexpr (CONV) {
            // a tap outside the image: the patch matrix holds zeros there
#pragma unroll
            for (int j = 0; j < 16; ++j) xh[j] = ring[b].valid[rt] ? xh[j] : 0.f;
          }
          if constexpr (MX) {
            quantize_mx(xh, packed, meta);
          } else {
            uint16_t s16;
            quantize_int4(xh, packed, s16);
            meta = s16;
          }
          if constexpr (NCB > 0) {
            // the lane's 16 values, rounded to fp16, are its two matrix
            // operands. Xhat is rounded to fp32 first and then to fp16 (RNE).
            // The conversion is written out: as plain code the backend folds
            // the product and the conversion into one v_fma_mixlo_f16, which
            // rounds only once and differs in rare double-rounding cases.
            v2h hp[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              uint32_t r;
              __asm__("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(xh[2 * j]), "v"(xh[2 * j + 1]));
              hp[j] = __builtin_bit_cast(v2h, r);
            }
            const v8h x0 = {hp[0][0], hp[0][1], hp[1][0], hp[1][1], hp[2][0], hp[2][1], hp[3][0], hp[3][1]};
            const v8h x1 = {hp[4][0], hp[4][1], hp[5][0], hp[5][1], hp[6][0], hp[6][1], hp[7][0], hp[7][1]};
            if constexpr (ring_l1_blocks<NCB>() > 0) {
#pragma unroll
              for (int c = 0; c < NCB; ++c) {
                acc[rt][c] = mfma_f16_16x16x32(x0, ring[b].l1[c][0], acc[rt][c]);
                acc[rt][c] = mfma_f16_16x16x32(x1, ring[b].l1[c][1], acc[rt][c]);
              }
            } else {
#pragma unroll
              for (int c = 0; c < NCB; ++c) {
                acc[rt][c] = mfma_f16_16x16x32(x0, *l1_operand(g, c, 0), acc[rt][c]);
                acc[rt][c] = mfma_f16_16x16x32(x1, *l1_operand(g, c, 1), acc[rt][c]);
              }
            }
          }
        }
        if constexpr (TILED) {
          // the row block exists (rows past M inside it carry the clamped
          // row's values, so the block is fully written)
          if (i < n_mine && row0 + 16 * rt < M) {
            const int64_t b = row0 / 16 + rt;
            *reinterpret_cast<v4i*>(a_codes + (b * G + g) * 1024 + 16 * lane) =
                widen_codes(make_uint2(packed[0], packed[1]));
            if (c4 == 0) {
              // the scale in fp32: row block i = b % 8 of its 128-row band, row
              // qr, at 64 (i/4) + 4 qr + i%4
              const int64_t ib = b % 8;
              static_cast<float*>(a_meta)[((b / 8) * G + g) * 128 + 64 * (ib / 4) + 4 * qr +
                                          ib % 4] = h2f(static_cast<uint16_t>(meta));
            }
          }
        } else if (i < n_mine && rvalid[rt]) {
          if constexpr (MX) {
            // tiled layouts: group g is half h of chunk g/2; this lane's 16
            // codes are the 8 bytes at 8*(c4%2) of lane 16*kq + qr of the
            // chunk's block, kq = 2h + c4/2 (its 32-block within the chunk);
            // the exponent of that 32-block (lanes c4 = 0, 2 hold the two) is
            // byte ti of lane 16*kq + qr of the chunk's exponent block
            const int c = g >> 1, h = g & 1;
            const int kq = 2 * h + (c4 >> 1);
            uint8_t* cb = tcode[rt] + static_cast<int64_t>(c) * 1024 + (16 * kq + qr) * 16 + 8 * (c4 & 1);
            uint8_t* eb = texp[rt] + static_cast<int64_t>(c) * 256 + (16 * kq + qr) * 4;
            *reinterpret_cast<uint2*>(cb) = make_uint2(packed[0], packed[1]);
            if ((c4 & 1) == 0) eb[0] = static_cast<uint8_t>(meta & 0xFFu);
            if (h == 0 && g == G - 1) {
              // K % 128 == 64: the chunk's second half does not exist; zero
              // codes and exponent 127 make it add exactly nothing
              *reinterpret_cast<uint2*>(cb + 32 * 16) = make_uint2(0u, 0u);
              if ((c4 & 1) == 0) eb[32 * 4] = 127;
            }
          } else {
            *reinterpret_cast<uint2*>(crow[rt] + g * kGroupBytes) = make_uint2(packed[0], packed[1]);
            if (c4 == 0) srow[rt][g] = static_cast<uint16_t>(meta);
          }
        }
      }
      // Refill this slot only after the stores: issued right behind the matrix
      // instructions that read the slot's L1 operands, the loads corrupted
      // some of those operands on gfx950 (D off by ~2e-5 relative).
      load_group(ring[b], i + NB);
    }
  }

  if constexpr (NCB > 0) {
    // partial D of this wave -> LDS; lane holds rows 4q+j of column c*16+rl
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int c = 0; c < NCB; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) dpart[wave][16 * rt + 4 * q + j][c * 16 + rl] = acc[rt][c][j];
    __syncthreads();
    for (int t = threadIdx.x; t < 16 * RT * R; t += blockDim.x) {
      const int r_ = t / R, c_ = t - r_ * R;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) s += dpart[w][r_][c_];
      if (SPLIT) {
        // the slice's partial: rows of all tiles (gridDim.x / S of them),
        // slice-major, fp32
        const int64_t rows_all = static_cast<int64_t>(gridDim.x / S) * (16 * RT);
        Dpart[(slice * rows_all + row0 + r_) * R + c_] = s;
      } else if (row0 + r_ < M) {
        if constexpr (TILED || MX) {
          // fp16(D) in the up-projection's operand order: per 16-row block
          // and 32-rank chunk one 1 KB block, lane 16q + r holding row r,
          // ranks 8q .. 8q+7 of the chunk (svdq.h, tiled layouts of both
          // formats)
          const int64_t m = row0 + r_;
          const int64_t blk = (m / 16) * ((R + 31) / 32) + c_ / 32;
          reinterpret_cast<uint16_t*>(D)[(blk * 64 + 16 * ((c_ % 32) / 8) + m % 16) * 8 + c_ % 8] =
              f2h(s);
        } else {
          D[(row0 + r_) * R + c_] = s;
        }
      }
    }
  }
}

// Sums the S partial D tiles of the split pre-kernel in slice order and writes
// fp16(D) in the up-projection's operand order (the tiled layouts' D_t): one
// lane per (16-row block, 32-rank chunk, lane 16q + r), i.e. row r, ranks
// 8q .. 8q+7 of the chunk, one 16-byte store.
__global__ __launch_bounds__(256) void k1_reduce_kernel(const float* __restrict__ part, int S,
                                                        int64_t rows_all, int64_t M, int R,
                                                        uint16_t* __restrict__ Dt) {
  const int RC = (R + 31) / 32;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t u = t >> 6;                       // (row block, rank chunk)
  const int lane = static_cast<int>(t & 63);
  const int64_t b = u / RC;
  const int c = static_cast<int>(u - b * RC);
  const int64_t m = 16 * b + (lane & 15);
  const int k = 32 * c + 8 * (lane >> 4);
  if (m >= M || k >= R) return;                   // R % 16 == 0: whole 8-runs are in or out
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int sl = 0; sl < S; ++sl) {
    const float4* p = reinterpret_cast<const float4*>(part + (sl * rows_all + m) * R + k);
    const float4 lo = p[0], hi = p[1];
    acc[0] += lo.x; acc[1] += lo.y; acc[2] += lo.z; acc[3] += lo.w;
    acc[4] += hi.x; acc[5] += hi.y; acc[6] += hi.z; acc[7] += hi.w;
  }
  uint4 o;
  o.x = f2h(acc[0]) | (static_cast<uint32_t>(f2h(acc[1])) << 16);
  o.y = f2h(acc[2]) | (static_cast<uint32_t>(f2h(acc[3])) << 16);
  o.z = f2h(acc[4]) | (static_cast<uint32_t>(f2h(acc[5])) << 16);
  o.w = f2h(acc[6]) | (static_cast<uint32_t>(f2h(acc[7])) << 16);
  *reinterpret_cast<uint4*>(Dt + ((b * RC + c) * 64 + lane) * 8) = o;
}

// S slices of the groups per row tile (S = 1: no split), and where the slices'
// partial D tiles go.
struct K1Split {
  int S;
  float* part;
};

template <typename XT, int NCB, int RT, int NB, int WV = k1_waves<NCB>()>
hipError_t launch_k1_rt(const void* X, int64_t M, int64_t K, int64_t ldx,
                        const float* inv_smooth, const uint16_t* L1p, int R,
                        uint8_t* a_codes, void* a_meta, int fmt, float* D, hipStream_t stream,
                        const ConvGeom* conv, K1Split sp = K1Split{1, nullptr}) {
  const int64_t tiles = (M + 16 * RT - 1) / (16 * RT);
  // only two-tile workgroups with one group in flight, on the tiled layouts of a
  // linear layer, have a split instance (the launch rule asks for no other)
  const bool split = RT == 2 && NB == 1 && NCB <= 6 && sp.S > 1 && conv == nullptr &&
                     fmt != kK1Int4;
  const dim3 block(64 * WV), grid(static_cast<unsigned>(tiles * (split ? sp.S : 1)));
  const XT* x = static_cast<const XT*>(X);
  const ConvGeom cg = conv ? *conv : ConvGeom{};
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, x, M, K, ldx, inv_smooth, L1p, R, a_codes,
                       a_meta, D, cg, sp.S, sp.part);
  };
  if constexpr (RT == 2 && NB == 1 && NCB <= 6) {
    if (split) {
      if (fmt == kK1Mx) go(k1_quant_down_kernel<XT, NCB, NB, kK1Mx, false, RT, WV, true>);
      else go(k1_quant_down_kernel<XT, NCB, NB, kK1Int4Tiled, false, RT, WV, true>);
      if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
      if (R > 0) {
        // every slice's partial is in place: sum them into D_t
        const int64_t units = ((M + 15) / 16) * ((R + 31) / 32);
        hipLaunchKernelGGL(k1_reduce_kernel,
                           dim3(static_cast<unsigned>((units * 64 + 255) / 256)), dim3(256), 0,
                           stream, sp.part, sp.S, tiles * 16 * RT, M, R,
                           reinterpret_cast<uint16_t*>(D));
      }
      return hipGetLastError();
    }
  }
  if (conv) {
    if (fmt == kK1Mx) go(k1_quant_down_kernel<XT, NCB, NB, kK1Mx, true, RT, WV>);
    else if (fmt == kK1Int4Tiled) go(k1_quant_down_kernel<XT, NCB, NB, kK1Int4Tiled, true, RT, WV>);
    else go(k1_quant_down_kernel<XT, NCB, NB, kK1Int4, true, RT, WV>);
  } else {
    if (fmt == kK1Mx) go(k1_quant_down_kernel<XT, NCB, NB, kK1Mx, false, RT, WV>);
    else if (fmt == kK1Int4Tiled) go(k1_quant_down_kernel<XT, NCB, NB, kK1Int4Tiled, false, RT, WV>);
    else go(k1_quant_down_kernel<XT, NCB, NB, kK1Int4, false, RT, WV>);
  }
  return hipGetLastError();
}

// Two row tiles per workgroup once there are more 16-row tiles than compute
// units (resident_slots() / 2), a row holds at least 16 groups of 64
// channels and the rank is at most 64. A row tile takes about the same time
// whatever else runs, so with 16-row workgroups some compute units would run
// two of them back to back; a 32-row workgroup costs less than that, and its
// waves share one set of smoothing factors and L1 operands. Each wave then
// keeps two groups in flight, three on long rows (at least 12 groups per
// wave) when every 32-row tile is resident at once. Measured inside the
// layer's step on MI355X (median of the pre-kernel's launches), against one
// 16-row tile per workgroup and one group in flight: DiT QKV 4608 x 3072 at
// rank 32 15.6-15.9 against 17.2-18.0 us, its MXFP4 version 15.3-15.5
// against 16.6-16.8 us; the 12288-channel down-projection at 4608 rows, three
// groups in flight against one: 41.0 against 46.1 us. Rows of fewer than 16
// groups keep 16-row tiles (32768 x 320: 11.8 against 12.7-13.2 us). At rank
// 96 (9216 x 3072) two tiles with two groups in flight were faster with X
// streamed from HBM alone but 1.3 us slower inside the step (42.6 against
// 41.3 us), so ranks above 64 keep 16-row tiles unless they are split (ranks
// 80 and 96 with a workspace: k1_slices). The convolution keeps its
// own rule (two tiles on patch matrices of more tiles than compute units
// unless the rows are short and every tile is resident: the 128 x 128 image
// took 48.0 against 56.1 us).
template <typename XT, int NCB>
hipError_t launch_k1_t(const void* X, int64_t M, int64_t K, int64_t ldx,
                       const float* inv_smooth, const uint16_t* L1p, int R,
                       uint8_t* a_codes, void* a_meta, int fmt, float* D, hipStream_t stream,
                       const ConvGeom* conv, float* part) {
  const int64_t tiles = (M + 15) / 16, slots = static_cast<int64_t>(resident_slots());
  const int64_t G = K / 64;
  if constexpr (NCB <= 4) {
    const bool all_resident = (M + 31) / 32 <= slots / 2;
    if (conv != nullptr) {
      const bool short_rows = G < 12 * k1_waves<NCB>() && tiles <= slots;
      if (2 * tiles > slots && !short_rows) {
        if (all_resident)
          return launch_k1_rt<XT, NCB, 2, 3>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta,
                                             fmt, D, stream, conv);
        return launch_k1_rt<XT, NCB, 2, 1>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt,
                                           D, stream, conv);
      }
    } else if (2 * tiles > slots && G >= 16) {
      const int S = k1_slices(M, K, R, fmt, false);
      if (S > 1 && (R == 0 || part != nullptr))
        return launch_k1_rt<XT, NCB, 2, 1>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt,
                                           D, stream, conv, K1Split{S, part});
      if (G >= 12 * k1_waves<NCB>() && all_resident)
        return launch_k1_rt<XT, NCB, 2, 3>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt,
                                           D, stream, conv);
      return launch_k1_rt<XT, NCB, 2, 2>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D,
                                         stream, conv);
    }
  } else if constexpr (NCB <= 6) {
    // ranks 80 and 96: 32-row tiles split along K, or 16-row tiles
    if (conv == nullptr && 2 * tiles > slots) {
      const int S = k1_slices(M, K, R, fmt, false);
      if (S > 1 && part != nullptr)
        return launch_k1_rt<XT, NCB, 2, 1>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt,
                                           D, stream, conv, K1Split{S, part});
    }
  }
  return launch_k1_rt<XT, NCB, 1, 1>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D,
                                     stream, conv);
}

template <typename XT>
hipError_t launch_k1_dtype(const void* X, int64_t M, int64_t K, int64_t ldx,
                                  const float* inv_smooth, const uint16_t* L1p, int R,
                                  uint8_t* a_codes, void* a_meta, int fmt, float* D,
                                  hipStream_t stream, const ConvGeom* conv, float* part) {
  switch (R / 16) {
    case 0: return launch_k1_t<XT, 0>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D, stream, conv, part);
    case 1: return launch_k1_t<XT, 1>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D, stream, conv, part);
    case 2: return launch_k1_t<XT, 2>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D, stream, conv, part);
    case 3: return launch_k1_t<XT, 3>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D, stream, conv, part);
    case 4: return launch_k1_t<XT, 4>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D, stream, conv, part);
    case 5: return launch_k1_t<XT, 5>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D, stream, conv, part);
    case 6: return launch_k1_t<XT, 6>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D, stream, conv, part);
    case 7:
    case 8: return launch_k1_t<XT, 8>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D, stream, conv, part);
    default: return launch_k1_t<XT, 16>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D, stream, conv, part);
  }
}

}  // namespace

hipError_t launch_k1(const void* X, bool x_f16, int64_t M, int64_t K, int64_t ldx,
                     const float* inv_smooth, const uint16_t* L1p, int R, uint8_t* a_codes,
                     void* a_meta, int fmt, float* D, hipStream_t stream, const ConvGeom* conv,
                     float* part) {
  if (x_f16)
    return launch_k1_dtype<_Float16>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D,
                                     stream, conv, part);
  return launch_k1_dtype<float>(X, M, K, ldx, inv_smooth, L1p, R, a_codes, a_meta, fmt, D, stream,
                                conv, part);
}

// Long rows (at least 12 groups per wave of a 32-row tile) with more 16-row
// tiles than compute units: each 32-row tile's groups are split over S
// workgroups, S = ceil(4 x compute units / 32-row tiles), at most G / 16, so
// that about four units of work per compute unit even out the tiles left
// over. Measured on MI355X on the 12288-channel down-projection at 4608 rows
// (144 tiles, S = 8), the pre-kernel alone with X streamed from HBM: 41.5 us
// plus 4 us for the reduction pass against 57.7 us unsplit.
// Ranks 80 and 96 are split whatever the row length: there the L1 operands
// (K x R fp16, 590 KB at 3072 x 96) are read again from L2 by every row tile,
// and 32-row tiles halve those reads; the split keeps the 32-row tiles from
// leaving compute units idle. Measured on MI355X on the 3072-channel LoRA
// layers at 9216 rows and rank 96 (288 tiles, S = 3), against 16-row tiles
// unsplit: pre-kernel 38.0 against 41.5 us, the 19-layer chain 3.40 against
// 3.58 ms in INT4 and 1.78 against 1.91 ms in MXFP4 (S = 2: 3.41 and 1.79 ms).
// The canonical layout (fp32 D), the convolution and ranks above 96 are not
// split.
int k1_slices(int64_t M, int64_t K, int R, int fmt, bool conv) {
  if (conv || fmt == kK1Int4 || R > 96 || M < 1 || K < 64) return 1;
  const int64_t tiles = (M + 15) / 16, slots = resident_slots(), G = K / 64;
  if (2 * tiles <= slots || (R <= 64 && G < 12 * 8)) return 1;
  const int64_t t32 = (M + 31) / 32, cus = slots / 2;
  int64_t S = (4 * cus + t32 - 1) / t32;
  if (S > G / 16) S = G / 16;
  return S < 2 ? 1 : static_cast<int>(S);
}

size_t k1_split_bytes(int64_t M, int64_t K, int R, int fmt, bool conv) {
  const int S = k1_slices(M, K, R, fmt, conv);
  if (S == 1 || R == 0) return 0;
  return static_cast<size_t>(S) * static_cast<size_t>((M + 31) / 32 * 32) *
         static_cast<size_t>(R) * 4;
}

}  // namespace svdq
