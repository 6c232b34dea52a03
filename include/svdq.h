/*
 * svdq.h -- C ABI of libsvdq, the SVDQuant W4A4 + low-rank linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (SVDQuant paper abstract as given on ai-digest.ru; chattools.cn
 * overview, section "SVDQuant的技术原理" (technical principles)):
 *
 *     Y = Xhat . L1 . L2  +  Q(Xhat) . Q(R)  +  b,      Xhat = X . diag(lam)^-1
 *
 * Smoothing moves activation outliers onto the weights; an SVD of the smoothed
 * weight diag(lam).W gives a 16-bit low-rank branch L1.L2 (rank R) and a
 * residual; the residual and Xhat are quantized to 4 bits with one fp16 scale
 * per group of 64 input channels. The inference-engine part of the pages
 * (the Nunchaku engine: the abstract, and the disruptive-concepts.com post,
 * section "Nunchaku: Fusing Precision and Speed") fuses the low-rank kernels
 * into the low-bit ones so the activation is not moved twice; here that is
 * two kernels:
 *
 *   K1  svdq_quantize_act_lowrank_down: one pass over X -> 4-bit codes,
 *       scales and the down-projection D = fp16(Xhat) . L1;
 *   K2  svdq_w4a4_gemm_lowrank_up: the W4A4 GEMM on the int8 matrix cores,
 *       integer partial sums per 64-channel group, fp32 rescale, and in the
 *       same kernel the up-projection fp16(D) . L2 and the bias.
 *
 * ---------------------------------------------------------------------------
 * Conventions (all functions)
 *   - Integer sizes are int64_t (shapes, strides) or int32_t (rank, group).
 *   - fp16 values travel as uint16_t bit patterns (IEEE binary16).
 *   - Return value: SVDQ_OK (0) or one SVDQ_ERR_* status. On an error nothing
 *     is launched and no output is written. No C++ exception crosses the ABI.
 *     svdq_last_error() (thread-local) then holds a one-line reason.
 *   - The caller owns every buffer. Device buffers must stay alive until the
 *     stream has completed the work that uses them.
 *   - NaN or Inf inputs give unspecified (but memory-safe) outputs.
 *
 * Canonical layouts (the bit-exact contract)
 *   - 4-bit codes are two's complement in [-7, 7]; element 2j is the low
 *     nibble of byte j, element 2j+1 the high nibble.
 *   - a_codes: M x K/2 bytes, row-major (row m holds token m along K).
 *     w_codes: N x K/2 bytes, row-major (row n holds output column n along K).
 *   - a_scales: M x K/group fp16, w_scales: N x K/group fp16, row-major.
 *   - The low-rank factors as the method states them (X . L1 . L2):
 *     L1: K x R fp16 row-major, L2: R x N fp16 row-major. svdq_linear_canonical
 *     takes them so; svdq_pack_lowrank turns them into the two packings the
 *     kernels read:
 *     L1p: L1 in K1's operand order (svdq_pack_lowrank_down gives the formula);
 *     L2t: N x R fp16 row-major (the transpose of L2), contiguous along the
 *     rank, which is what a matrix-core operand lane loads.
 *     The offline preparation writes L1t (R x K, the transpose of L1) and L2t.
 *   - D: M x R fp32 row-major.  X: M x K row-major with row stride ldx
 *     (elements).  Y: M x N row-major with row stride ldy (elements).
 *
 * Quantizer (the pages give only "4 bits"; this is the reading implemented,
 * for both Xhat rows and residual columns, over each group v of 64 values):
 *     a = max|v|;  s = fp16_rne(min(fp32(a / 7), 65504));
 *     inv = (s == 0) ? 0 : fp32(1 / s);  q = clamp(rint(fp32(v * inv)), -7, 7)
 * with correctly rounded fp32 division and multiplication and rounding half to
 * even. Xhat = fp32(x * inv_smooth[k]).
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVDQ_ABI_VERSION 12

/* status codes */
enum {
  SVDQ_OK = 0,
  SVDQ_ERR_NULL = 1,       /* a required pointer is NULL */
  SVDQ_ERR_SHAPE = 2,      /* a size or stride is out of range */
  SVDQ_ERR_ALIGN = 3,      /* a device pointer or row stride is not 16-byte aligned */
  SVDQ_ERR_DTYPE = 4,      /* unknown dtype code */
  SVDQ_ERR_RANK = 5,       /* rank out of range or not a multiple of 16 */
  SVDQ_ERR_WORKSPACE = 6,  /* workspace too small */
  SVDQ_ERR_HIP = 7,        /* a HIP call failed; svdq_last_error() has its message */
  SVDQ_ERR_NO_DEVICE = 8,  /* no usable GPU */
  SVDQ_ERR_INTERNAL = 9,   /* host numerical routine failed (e.g. no convergence) */
  SVDQ_ERR_GROUP = 10,     /* group size other than 64, or K not a multiple of it */
  SVDQ_ERR_ACT = 11        /* unknown activation code */
};

/* dtype codes for X and Y */
enum { SVDQ_F16 = 1, SVDQ_F32 = 2 };

/* Activation applied by K2's epilogue to the fp32 result before its one
 * rounding to the output type. GELU is the tanh form between the two linears
 * of a DiT MLP (not on the pages: the textbook formula, as in
 * svdq_gelu_tanh_f16), fused here so the intermediate is written once. */
enum { SVDQ_ACT_NONE = 0, SVDQ_ACT_GELU_TANH = 1 };

/* The only group size implemented. */
#define SVDQ_GROUP 64
/* Values per shared scale in the MXFP4 format. */
#define SVDQ_MX_BLOCK 32
/* Largest rank the device kernels accept. */
#define SVDQ_MAX_RANK 256

/* ---------------------------------------------------------------------------
 * Utilities
 */
int svdq_abi_version(void);
const char* svdq_status_str(int status);
/* Reason for the last non-OK status returned on this thread ("" if none). */
const char* svdq_last_error(void);

/* ---------------------------------------------------------------------------
 * Host functions: pointers are host memory; synchronous; thread-safe; no
 * global state. They never touch a GPU.
 */

/* out[k] = max over the M rows of |X[m][k]|.  X: M x K, row stride ldx >= K.
 * Calibration statistic for the smoothing factors. */
int svdq_channel_absmax(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                        float* out);

/* Smoothing factors (chattools.cn overview, technical principles, outlier
 * item: activation outliers are moved onto the weights).
 *   lambda[j] = fp32( sqrt( x_absmax[j] / max_n |W[j][n]| ) ), computed in fp64,
 *   and 1 where either maximum is 0 (migration strength 1/2).
 * W: K x N row-major fp32 (Y = X . W). */
int svdq_smoothing_factors(const float* x_absmax, const float* W, int64_t K, int64_t N,
                           float* lambda);

/* Offline weight preparation (chattools.cn overview, technical principles:
 * smoothing, SVD into a 16-bit low-rank branch and a residual, 4-bit residual;
 * the Eckart-Young-Mirsky item for the choice of the top singular values).
 *   inv_smooth[k] = fp32(1 / lambda[k])
 *   What = diag(lambda) . W (fp64), What = U S V^T (top `rank` triplets, fp64;
 *     the entry of largest magnitude of each u_i is made positive)
 *   L1 = fp16(U_r S_r^(1/2)) written as L1t (rank x K);
 *   L2 = fp16(S_r^(1/2) V_r^T) written as L2t (N x rank);
 *   R  = What - L1 . L2 from the stored fp16 factors (fp64), then fp32;
 *   w_codes / w_scales = the quantizer applied down K for each column n.
 *   sigma (optional, may be NULL): all min(K, N) singular values of What,
 *   descending.
 * Constraints: K % 64 == 0, group == 64, 0 <= rank <= min(K, N), N >= 1.
 * rank need not be a multiple of 16 here, but the device kernels require it.
 * Uses OpenMP threads. Returns SVDQ_ERR_INTERNAL if the eigen-solver fails. */
int svdq_prepare_weights(const float* W, const float* lambda, int64_t K, int64_t N,
                         int32_t rank, int32_t group, float* inv_smooth, uint16_t* L1t,
                         uint16_t* L2t, uint8_t* w_codes, uint16_t* w_scales, double* sigma);

/* Offline weight preparation for the MXFP4 format (see "MXFP4 format" below):
 * the same inv_smooth, SVD split, L1t, L2t and sigma as svdq_prepare_weights,
 * then the fp32 residual R in MXFP4 down K for each output column n:
 *   w_codes: N x K/2 bytes (E2M1 codes, element 2j in the low nibble),
 *   w_e8m0:  N x K/32 bytes (shared exponents, biased by 127).
 * Constraints: K % 64 == 0, 0 <= rank <= min(K, N), N >= 1. */
int svdq_prepare_weights_mx(const float* W, const float* lambda, int64_t K, int64_t N,
                            int32_t rank, float* inv_smooth, uint16_t* L1t, uint16_t* L2t,
                            uint8_t* w_codes, uint8_t* w_e8m0, double* sigma);

/* LoRA concatenation without re-quantization (chattools.cn overview, main
 * features, LoRA item; SVDQuant abstract). The branch multiplies Xhat, so row
 * j of A is scaled by lambda[j]:  Xhat . (lambda (.) A) = X . A.
 *   L1' = [L1 | fp16(lambda (.) A * scale)]   written as L1t_out ((rank+rl) x K)
 *   L2' = [L2 ; B]                             written as L2t_out (N x (rank+rl))
 * The product lambda*A is exact in fp64, the scale multiply rounds once in
 * fp64, the result rounds once to fp16. A: K x rl fp16, B: rl x N fp16 (both
 * row-major, the usual LoRA down/up shapes). w_codes and w_scales are reused
 * unchanged. Inputs and outputs must not overlap. */
int svdq_concat_lora(const uint16_t* L1t, const uint16_t* L2t, int64_t K, int64_t N,
                     int32_t rank, const float* lambda, const uint16_t* A, const uint16_t* B,
                     int32_t rl, float scale, uint16_t* L1t_out, uint16_t* L2t_out);

/* The low-rank down-projection factor in the order K1 consumes it (a layout,
 * no arithmetic). K1 feeds fp16(Xhat) to the matrix instruction
 * v_mfma_f32_16x16x32_f16 as two operands per 64-channel group, lane
 * l = 16*q + rl holding row rl and channels 16*q + 8*h .. +7 for h = 0, 1.
 * The matching L1 operands are stored so that each is one contiguous 1 KB
 * run (64 lanes x 8 fp16):
 *   L1p[(((g * R/16 + c) * 2 + h) * 64 + 16*q + rl) * 8 + j]
 *     = L1t[(16*c + rl) * K + 64*g + 16*q + 8*h + j]
 * for group g < K/64, column block c < R/16, h < 2, q < 4, rl < 16, j < 8.
 * L1t: R x K fp16 (as written by svdq_prepare_weights / svdq_concat_lora);
 * L1p: R*K fp16. K % 64 == 0, 16 <= R <= SVDQ_MAX_RANK, R % 16 == 0. */
int svdq_pack_lowrank_down(const uint16_t* L1t, int64_t K, int32_t R, uint16_t* L1p);

/* The canonical low-rank factors -> the device packings (a layout, no
 * arithmetic): L1 (K x R fp16, row-major) -> L1p as svdq_pack_lowrank_down
 * writes it (L1p[...] = L1[64g + 16q + 8h + j][16c + rl] in its formula), and
 * L2 (R x N fp16, row-major) -> L2t[n][r] = L2[r][n] (N x R). The factors are
 * those of the 16-bit low-rank branch of the SVD split (chattools.cn overview,
 * section "SVDQuant的技术原理"). K % 64 == 0, N >= 1, 16 <= R <= SVDQ_MAX_RANK,
 * R % 16 == 0. Outputs must not overlap inputs. */
int svdq_pack_lowrank(const uint16_t* L1, const uint16_t* L2, int64_t K, int64_t N, int32_t R,
                      uint16_t* L1p, uint16_t* L2t);

/* ---------------------------------------------------------------------------
 * Device functions: pointers are device memory; the work is enqueued on
 * `stream` (0 = the null stream) and the call returns without waiting. They
 * never allocate device memory and never synchronize.
 * Common constraints: M >= 1, N >= 1, K >= 64 with K % 64 == 0, group == 64,
 * 0 <= R <= SVDQ_MAX_RANK with R % 16 == 0; K <= ldx <= 2^25, ldy >= N.
 * Alignment: X, inv_smooth, L1p, L2t, D, codes and scales 16 bytes, and
 * ldx * sizeof(X element) a multiple of 16 bytes (X rows are read in 16-byte
 * vectors); Y and bias only to their element size, any ldy.
 */

/* K1: one pass over X (SVDQuant abstract: fuse the low-rank branch with the
 * low-bit kernels so the activation is not moved again).
 *   Xhat = fp32(x * inv_smooth[k]);
 *   a_codes, a_scales = the quantizer over each row's groups of 64;
 *   D = fp16(Xhat) . L1   (fp16 products, fp32 accumulation), D: M x R.
 * L1p: L1 packed by svdq_pack_lowrank_down. With R == 0, L1p and D may be NULL. */
int svdq_quantize_act_lowrank_down(const void* X, int x_dtype, int64_t M, int64_t K,
                                   int64_t ldx, const float* inv_smooth, const uint16_t* L1p,
                                   int32_t R, int32_t group, uint8_t* a_codes,
                                   uint16_t* a_scales, float* D, hipStream_t stream);

/* K2: W4A4 GEMM with the low-rank up-projection and bias fused in. Both
 * operands 4-bit (SVDQuant abstract, ai-digest.ru page: weights and
 * activations quantized to 4 bits); the low-rank branch's second product runs
 * inside the low-bit GEMM rather than as a kernel of its own (the Nunchaku
 * engine fuses the low-rank kernels into the low-bit ones: chattools.cn
 * overview, section "SVDQuant的技术原理", Nunchaku item; disruptive-concepts.com
 * post, section "Nunchaku: Fusing Precision and Speed").
 *   P[m,n,g] = sum over k in group g of qx[m,k] * qw[n,k]   (exact int32)
 *   Y[m,n]   = sum_g s_x[m,g] * s_w[n,g] * P[m,n,g]   (fp32)
 *              + sum_r fp16(D[m,r]) * L2[r,n]          (fp16 products, fp32 sum)
 *              + bias[n]                               (bias may be NULL)
 * then the activation (SVDQ_ACT_*) in fp32, rounded once to y_dtype.
 * With R == 0, D and L2t may be NULL. */
int svdq_w4a4_gemm_lowrank_up(const uint8_t* a_codes, const uint16_t* a_scales,
                              const uint8_t* w_codes, const uint16_t* w_scales, const float* D,
                              const uint16_t* L2t, int32_t R, const float* bias, void* Y,
                              int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy,
                              int32_t group, int32_t activation, hipStream_t stream);

/* Bytes of workspace svdq_linear needs: a_codes, a_scales and D, each
 * 256-byte aligned inside the workspace. */
size_t svdq_linear_workspace_bytes(int64_t M, int64_t K, int32_t R, int32_t group);

/* The whole layer Y = Xhat . L1 . L2 + Q(Xhat) . Q(R) + b (chattools.cn
 * overview, section "SVDQuant的技术原理": the low-rank branch beside the 4-bit
 * residual branch), as the Nunchaku engine runs it: two kernels, the low-rank
 * down-projection fused into the activation quantizer and the up-projection
 * into the W4A4 GEMM (chattools.cn overview, Nunchaku item; disruptive-
 * concepts.com post, section "Nunchaku: Fusing Precision and Speed"; the
 * SVDQuant abstract: the activation is not moved a second time). K1 then K2 on
 * `stream`, intermediates in `ws` (>= svdq_linear_workspace_bytes(M, K, R,
 * group) bytes, 256-byte aligned). L1p: packed by svdq_pack_lowrank_down or
 * svdq_pack_lowrank, L2t: N x R. activation: SVDQ_ACT_*. */
int svdq_linear(const void* X, int x_dtype, int64_t ldx, const float* inv_smooth,
                const uint16_t* L1p, const uint16_t* L2t, int32_t R, const uint8_t* w_codes,
                const uint16_t* w_scales, const float* bias, void* Y, int y_dtype, int64_t ldy,
                int64_t M, int64_t K, int64_t N, int32_t group, void* ws, size_t ws_bytes,
                int32_t activation, hipStream_t stream);

/* Bytes of workspace svdq_linear_canonical needs: svdq_linear's, then room
 * for the packed factors (R*K and N*R fp16), each 256-byte aligned. */
size_t svdq_linear_canonical_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t R,
                                             int32_t group);

/* svdq_linear taking the low-rank factors as the method states them: L1
 * (K x R) and L2 (R x N), fp16 row-major device arrays (the SVD split of the
 * smoothed weight into a 16-bit low-rank branch and a 4-bit residual:
 * chattools.cn overview, section "SVDQuant的技术原理"). A layout kernel first
 * writes L1p and L2t into `ws` (>= svdq_linear_canonical_workspace_bytes),
 * then the same K1 and K2 as svdq_linear: the result is bit-identical to
 * svdq_linear on the packed factors. The packing is repeated on every call;
 * callers that run a layer many times pack once (svdq_pack_lowrank) and call
 * svdq_linear. L1, L2: 16-byte aligned; may be NULL when R == 0. */
int svdq_linear_canonical(const void* X, int x_dtype, int64_t ldx, const float* inv_smooth,
                          const uint16_t* L1, const uint16_t* L2, int32_t R,
                          const uint8_t* w_codes, const uint16_t* w_scales, const float* bias,
                          void* Y, int y_dtype, int64_t ldy, int64_t M, int64_t K, int64_t N,
                          int32_t group, void* ws, size_t ws_bytes, int32_t activation,
                          hipStream_t stream);

/* Largest intermediate size svdq_linear_noalloc handles (bytes of
 * svdq_linear_workspace_bytes): 64 MiB, enough for every layer shape used
 * here (the DiT MLP down-projection needs 31 MB, the largest UNet
 * convolution 54 MB). */
#define SVDQ_NOALLOC_MAX_BYTES (64u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): svdq_linear
 * with its intermediates (activation codes, scales, D) in a static device
 * buffer of SVDQ_NOALLOC_MAX_BYTES that the library holds on each GPU it runs
 * on until the process ends, instead of a caller workspace. Same arguments,
 * results and checks as svdq_linear otherwise. Returns SVDQ_ERR_WORKSPACE (and
 * launches nothing) when svdq_linear_workspace_bytes(M, K, R, group) exceeds
 * the buffer. It calls no allocator. Every call on one GPU shares that GPU's
 * buffer: calls that overlap on one GPU (other streams, other threads) race
 * and must be serialized by the caller. */
int svdq_linear_noalloc(const void* X, int x_dtype, int64_t ldx, const float* inv_smooth,
                        const uint16_t* L1p, const uint16_t* L2t, int32_t R,
                        const uint8_t* w_codes, const uint16_t* w_scales, const float* bias,
                        void* Y, int y_dtype, int64_t ldy, int64_t M, int64_t K, int64_t N,
                        int32_t group, int32_t activation, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Tiled INT4 path: the same layer, the same codes, scales and arithmetic as
 * svdq_linear (the fused pre-kernel and the W4A4 GEMM with the low-rank
 * up-projection in its epilogue: SVDQuant abstract on ai-digest.ru;
 * chattools.cn overview, section "SVDQuant的技术原理", Nunchaku item), with the
 * operands laid out so the GEMM spends its vector ALU on the per-group
 * rescale alone. Layouts, with G = K/64 groups:
 *   a_ops_t   activation operands, ceil(M/16) x G blocks of 1024 bytes; block
 *             (b, g) lane l = 16q + r (q < 4, r < 16) holds 16 int8 bytes:
 *             with c_j the code of row 16b + r at k = 64g + 16q + j, bytes
 *             0..3 = 16*(c0, c2, c4, c6), 4..7 = 16*(c1, c3, c5, c7),
 *             8..11 = 16*(c8, c10, c12, c14), 12..15 = 16*(c9, c11, c13, c15).
 *             Rows past M inside the last block hold row M-1's values.
 *   a_scales_t activation scales, ceil(M/128) x G blocks of 128 fp32; block
 *             (t, g) holds s = fp32(the fp16 group scale) of row 128t + 16i + r
 *             (i < 8, r < 16) at index 64*(i/4) + 4r + i%4.
 *   w_codes_t weight codes, 4-bit as in the canonical layout, ceil(N/32) x G
 *             blocks of 1024 bytes; block (s, g) lane l = 16q + r holds bytes
 *             32g + 8q .. +7 of the canonical rows of columns 32s + r (bytes
 *             0..7) and 32s + 16 + r (bytes 8..15); 0 past N.
 *   w_scales_t weight scales as fp32 pairs, ceil(N/32) x G blocks of 64 fp32;
 *             entries 16q + 8j + 2e and 16q + 8j + 2e + 1 of block (s, g) are
 *             (s/256, -12582912 s/256), s = fp32(the fp16 scale of column
 *             32s + 16j + 4q + e in group g), both exact; 0 past N. The pair
 *             turns the matrix instruction's biased result into P s exactly.
 *   D_t       the down-projection D in fp16 (rounded once from its fp32
 *             sum, as the up-projection of K2 rounds it), ceil(M/16) x
 *             ceil(R/32) blocks of 512 fp16; element 8l + j of block (b, c),
 *             lane l = 16q + r, is fp16(D[16b + r][32c + 8q + j]). Entries past
 *             M or past R are not written and not read.
 * The weight layouts are a permutation of the canonical w_codes / w_scales
 * (svdq_pack_w4a4_tiles), made once offline; the weights stay at 4 bits.
 */

/* Bytes of the tiled INT4 layouts (0 for invalid sizes). */
size_t svdq_int4_act_tiled_bytes(int64_t M, int64_t K);
size_t svdq_int4_act_scales_tiled_bytes(int64_t M, int64_t K);
size_t svdq_int4_d_tiled_bytes(int64_t M, int32_t R);
size_t svdq_int4_w_codes_tiled_bytes(int64_t N, int64_t K);
size_t svdq_int4_w_scales_tiled_bytes(int64_t N, int64_t K);

/* Host: canonical w_codes (N x K/2) and w_scales (N x K/64 fp16) -> the tiled
 * weight layouts above (a permutation of the codes, the scales as exact fp32
 * pairs, zero padding). K % 64 == 0, N >= 1. Outputs must not overlap inputs. */
int svdq_pack_w4a4_tiles(const uint8_t* w_codes, const uint16_t* w_scales, int64_t N, int64_t K,
                         uint8_t* w_codes_t, float* w_scales_t);

/* Bytes of the optional workspace of the tiled and MXFP4 pre-kernels
 * (svdq_quantize_act_lowrank_down_tiled, _mx) for this shape on the current
 * device: on long rows (at least 96 groups of 64, more 16-row tiles than
 * compute units, R <= 64) the pre-kernel splits each 32-row tile's groups
 * over several workgroups and needs room for their fp32 partial D tiles,
 * which a second pass sums in a fixed order into D_t (SVDQuant abstract on
 * ai-digest.ru: the fused low-rank branch must not cost the layer its
 * speed; the split evens out row tiles that do not divide over the compute
 * units). 0 when the shape is not split, or R == 0 (no D), or the sizes are
 * invalid. */
size_t svdq_quantize_act_workspace_bytes(int64_t M, int64_t K, int32_t R);

/* Device: K1 (svdq_quantize_act_lowrank_down: the same smoothing, quantizer
 * and D) writing the codes, scales and D as a_ops_t, a_scales_t and D_t
 * (svdq_int4_act_tiled_bytes(M, K), svdq_int4_act_scales_tiled_bytes(M, K) and
 * svdq_int4_d_tiled_bytes(M, R) bytes, 16-byte aligned; D_t may be NULL when
 * R == 0). workspace: NULL, or at least svdq_quantize_act_workspace_bytes(M,
 * K, R) bytes, 256-byte aligned (else SVDQ_ERR_WORKSPACE / SVDQ_ERR_ALIGN);
 * with it a shape that splits runs split (its D_t sums the same terms in
 * another order, within the same bound), without it unsplit. The codes and
 * scales are the same either way. */
int svdq_quantize_act_lowrank_down_tiled(const void* X, int x_dtype, int64_t M, int64_t K,
                                         int64_t ldx, const float* inv_smooth,
                                         const uint16_t* L1p, int32_t R, uint8_t* a_ops_t,
                                         float* a_scales_t, uint16_t* D_t, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/* Bytes of the tiled GEMM's optional workspace for this shape on the current
 * device: when its 128 x 128 tiles fill at most a quarter of the resident
 * workgroup slots and K holds at least 32 groups (an under-filled long-K
 * GEMM, e.g. the UNet's 32x32 convolution), every tile is split along K over
 * several workgroups whose fp32 partial tiles a second pass sums in slice
 * order before the bias, the activation and the rounding. 0 when the shape is
 * not split or the sizes are invalid. */
size_t svdq_gemm_tiled_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Device: K2 (svdq_w4a4_gemm_lowrank_up: the same exact int32 group partials,
 * fp32 rescale, low-rank up-projection, bias and activation) on the tiled
 * layouts. The order of the fp32 sums differs from K2's (the low-rank term
 * first), within the same rounding bound. workspace: NULL, or at least
 * svdq_gemm_tiled_workspace_bytes(M, N, K) bytes, 256-byte aligned (else
 * SVDQ_ERR_WORKSPACE / SVDQ_ERR_ALIGN); with it a shape that splits runs split
 * along K (the same sums in another order, within the same bound), without it
 * unsplit. */
int svdq_w4a4_gemm_lowrank_up_tiled(const uint8_t* a_ops_t, const float* a_scales_t,
                                    const uint8_t* w_codes_t, const float* w_scales_t,
                                    const uint16_t* D_t, const uint16_t* L2t, int32_t R,
                                    const float* bias, void* Y, int y_dtype, int64_t M, int64_t N,
                                    int64_t K, int64_t ldy, int32_t activation, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace svdq_linear_tiled needs on the current device: a_ops_t,
 * a_scales_t, D_t and the split pre-kernel's partial D tiles (see
 * svdq_quantize_act_workspace_bytes), each 256-byte aligned inside the
 * workspace. */
size_t svdq_linear_tiled_workspace_bytes(int64_t M, int64_t K, int32_t R);

/* The whole layer on the tiled path: the tiled K1 then the tiled K2 on
 * `stream`, intermediates in `ws` (256-byte aligned); the weights tiled by
 * svdq_pack_w4a4_tiles. When `ws` holds svdq_gemm_tiled_workspace_bytes(M, N,
 * K) more bytes after svdq_linear_tiled_workspace_bytes(M, K, R), an
 * under-filled GEMM runs split along K there. */
int svdq_linear_tiled(const void* X, int x_dtype, int64_t ldx, const float* inv_smooth,
                      const uint16_t* L1p, const uint16_t* L2t, int32_t R,
                      const uint8_t* w_codes_t, const float* w_scales_t, const float* bias,
                      void* Y, int y_dtype, int64_t ldy, int64_t M, int64_t K, int64_t N,
                      void* ws, size_t ws_bytes, int32_t activation, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * MXFP4 format (the CDNA4 counterpart of the 4-bit floating-point version of
 * the method that the taicenter.com news page names for the newest hardware,
 * section on hardware co-design for Blackwell GPUs, NVFP4 item; the pages give
 * no format details). Reading implemented, after OCP "Microscaling Formats
 * (MX) Specification" v1.0, for Xhat rows and residual columns alike, over
 * each block v of 32 consecutive values along K:
 *     e = max(floor(log2(max|v|)) - 2, -127)   (-127 for an all-zero block;
 *         as a byte: the biased exponent field of max|v| minus 2, floored at 0)
 *     E8M0 byte = e + 127;  code = E2M1 nearest to v / 2^e, ties to the even
 *     code, magnitudes above 6 saturating to 6, sign bit kept (-0 is code 8)
 * E2M1 codes s e1 e0 m: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for m|e = 0..7,
 * bit 3 the sign; two per byte, element 2j in the low nibble.
 * Canonical layouts (host side, as svdq_prepare_weights_mx writes them):
 * codes rows x K/2 bytes and E8M0 exponents rows x K/32 bytes, row-major.
 *
 * Tiled layouts (device side, what K1-MX writes and K2-MX reads): each load of
 * the matrix instruction's operands becomes one contiguous run. With
 * C = ceil(K/128) chunks of 128 values along K:
 *   codes_t: ceil(rows/16) x C blocks of 1024 bytes; in block (b, c) lane
 *     l = 16*q + r (q < 4, r < 16) holds bytes 16*l .. 16*l+15 =
 *     canonical codes of row 16*b + r, bytes 64*c + 16*q .. +15;
 *   exps_t: ceil(rows/64) x C blocks of 256 bytes; in block (g, c) byte
 *     4*l + i (l = 16*q + r, i < 4) = E8M0 of row 64*g + 16*i + r, 32-block
 *     4*c + q.
 * Entries past the last row or past K (the second half of the last chunk when
 * K % 128 == 64) hold zero codes and exponent 127 where svdq_pack_mx_tiles
 * writes them; K1-MX writes the entries past K the same way and leaves rows
 * past M unwritten (K2-MX never stores the outputs that depend on them).
 * Smoothing and the low-rank factors are as in the INT4 functions; D travels
 * from K1-MX to K2-MX as D_t, fp16 in the up-projection's operand order, as on
 * the tiled INT4 path (svdq_int4_d_tiled_bytes(M, R) bytes, 16-byte aligned).
 * Constraints and alignment as for the device functions above (the tiled
 * arrays 16-byte aligned); K % 64 == 0. */

/* Bytes of the tiled layouts for `rows` rows of length K (0 for invalid sizes). */
size_t svdq_mx_codes_tiled_bytes(int64_t rows, int64_t K);
size_t svdq_mx_exps_tiled_bytes(int64_t rows, int64_t K);

/* Host: canonical codes (rows x K/2) and exponents (rows x K/32) -> the tiled
 * layouts above, padding included (a permutation, no arithmetic). Used for the
 * weights, whose tiles are made once offline. Outputs must not overlap inputs. */
int svdq_pack_mx_tiles(const uint8_t* codes, const uint8_t* e8m0, int64_t rows, int64_t K,
                       uint8_t* codes_t, uint8_t* exps_t);

/* K1-MX: as svdq_quantize_act_lowrank_down with the MXFP4 quantizer; a_codes_t
 * and a_exps_t in the tiled layouts (svdq_mx_*_tiled_bytes(M, K) bytes); D as
 * D_t (fp16 D in operand order, the layout of the tiled INT4 path; NULL when
 * R == 0). workspace: as for svdq_quantize_act_lowrank_down_tiled (the same
 * svdq_quantize_act_workspace_bytes). */
int svdq_quantize_act_lowrank_down_mx(const void* X, int x_dtype, int64_t M, int64_t K,
                                      int64_t ldx, const float* inv_smooth, const uint16_t* L1p,
                                      int32_t R, uint8_t* a_codes_t, uint8_t* a_exps_t,
                                      uint16_t* D_t, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* K2-MX: Y[m,n] = sum_k deq(a)[m,k] * deq(w)[n,k] (products and sums in the
 * matrix core's fp32 accumulation, deq = E2M1 value * 2^e of its block)
 *                 + sum_r fp16(D[m,r]) * L2[r,n] + bias[n]
 * then the activation (SVDQ_ACT_*) in fp32, rounded once to y_dtype.
 * All four code and exponent arrays in the tiled layouts; fp16(D) as D_t, as
 * K1-MX writes it. */
int svdq_mx_gemm_lowrank_up(const uint8_t* a_codes_t, const uint8_t* a_exps_t,
                            const uint8_t* w_codes_t, const uint8_t* w_exps_t, const uint16_t* D_t,
                            const uint16_t* L2t, int32_t R, const float* bias, void* Y,
                            int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy,
                            int32_t activation, hipStream_t stream);

/* Bytes of workspace svdq_linear_mx needs on the current device: the tiled
 * activation codes and exponents, D_t and the split pre-kernel's partial D
 * tiles, each 256-byte aligned inside the workspace (0 for invalid sizes). */
size_t svdq_linear_mx_workspace_bytes(int64_t M, int64_t K, int32_t R);

/* The whole MXFP4 layer: K1-MX then K2-MX on `stream`, intermediates in `ws`;
 * the weights in the tiled layouts. */
int svdq_linear_mx(const void* X, int x_dtype, int64_t ldx, const float* inv_smooth,
                   const uint16_t* L1p, const uint16_t* L2t, int32_t R, const uint8_t* w_codes_t,
                   const uint8_t* w_exps_t, const float* bias, void* Y, int y_dtype, int64_t ldy,
                   int64_t M, int64_t K, int64_t N, void* ws, size_t ws_bytes,
                   int32_t activation, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * 4-bit weight-only baseline (W4A16): the comparison baseline of the SVDQuant
 * abstract (ai-digest.ru page: 3.0x faster than a 4-bit weight-only baseline),
 * which gives no format. Reading implemented: the quantizer above applied to W
 * itself (per output column, groups of 64 along K; no smoothing, no low-rank
 * branch), fp16 activations, each weight dequantized to fp16(s * q) with one
 * rounding, fp32 accumulation:
 *     Y = fp16(X) . fp16(s q)^T + bias, rounded once to y_dtype.
 *
 * Tiled device layouts (S = K/32 steps of 32 along K, G = K/64 groups):
 *   x_t:      ceil(M/16) x S blocks of 1024 bytes (fp16): in block (b, s) lane
 *             l = 16q + r holds 8 fp16 of row 16b + r at k = 32s + 8q + e,
 *             in the order e = 0, 4, 1, 5, 2, 6, 3, 7;
 *   codes_t:  ceil(N/16) x S blocks of 256 bytes: in block (b, s) lane l holds
 *             the 4 bytes 16s + 4q .. +3 of column 16b + r (8 codes, element
 *             2j in the low nibble of byte j), each nibble stored as code + 8;
 *   scales_t: ceil(N/64) x G blocks of 64 fp16: entry 4r + j of block (c, g)
 *             is the scale of column 64c + 16j + r in group g.
 * Entries past N hold code 0 (stored as 8) and scale 0.
 */

/* Host: w_codes (N x K/2) and w_scales (N x K/64 fp16) = the quantizer on W
 * (K x N fp32, Y = X . W), canonical layout. K % 64 == 0, N >= 1. */
int svdq_prepare_weights_w4a16(const float* W, int64_t K, int64_t N, uint8_t* w_codes,
                               uint16_t* w_scales);

/* Bytes of the tiled weight layouts (0 for invalid sizes). */
size_t svdq_w4a16_codes_tiled_bytes(int64_t N, int64_t K);
size_t svdq_w4a16_scales_tiled_bytes(int64_t N, int64_t K);

/* Host: canonical W4A16 weights -> the tiled layouts above (a permutation,
 * and the +8 of the stored codes). Outputs must not overlap inputs. */
int svdq_pack_w4a16_tiles(const uint8_t* w_codes, const uint16_t* w_scales, int64_t N, int64_t K,
                          uint8_t* codes_t, uint16_t* scales_t);

/* Bytes of the tiled fp16 activation (0 for invalid sizes). */
size_t svdq_w4a16_x_tiled_bytes(int64_t M, int64_t K);

/* Device: X (M x K fp16 or fp32, row stride ldx) -> x_t, the tiled fp16 layout
 * above (fp32 values rounded to fp16, RNE). Rows past M in the last block are
 * copies of row M-1. Constraints as for K1 (X 16-byte aligned rows). */
int svdq_w4a16_tile_activation(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                               uint16_t* x_t, hipStream_t stream);

/* Device: Y = x . deq(w)^T + bias on the tiled layouts, one rounding to y_dtype. */
int svdq_w4a16_gemm(const uint16_t* x_t, const uint8_t* w_codes_t, const uint16_t* w_scales_t,
                    const float* bias, void* Y, int y_dtype, int64_t M, int64_t N, int64_t K,
                    int64_t ldy, hipStream_t stream);

/* Device: the whole baseline layer (tiling of X into `ws`, then the GEMM);
 * ws >= svdq_w4a16_x_tiled_bytes(M, K) bytes, 256-byte aligned. */
int svdq_linear_w4a16(const void* X, int x_dtype, int64_t ldx, const uint8_t* w_codes_t,
                      const uint16_t* w_scales_t, const float* bias, void* Y, int y_dtype,
                      int64_t ldy, int64_t M, int64_t K, int64_t N, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Convolutions (the chattools.cn overview, section "SVDQuant的技术原理", says
 * the method serves UNet backbones as well as DiT ones; the pages give no
 * convolution-specific rule). Reading implemented: a KH x KW convolution with
 * square stride and zero padding is the linear layer above on its patch
 * matrix, with no patch matrix in memory:
 *   X      NHWC image, batch x H x W x C, contiguous, fp16 or fp32;
 *          C a positive multiple of 64 (a group of 64 never straddles taps);
 *   M = batch * OH * OW patches (row p = (b, oh, ow), b-major),
 *          OH = (H + 2 pad - KH) / stride + 1, OW likewise;
 *   K = KH * KW * C, column (kh * KW + kw) * C + c holding channel c of pixel
 *          (oh * stride + kh - pad, ow * stride + kw - pad), 0 outside the image;
 *   lam, L1, L2, the residual: those of the K x N weight matrix Wm whose row
 *          (kh * KW + kw) * C + c is the filter tap (kh, kw, c), i.e. a
 *          KH x KW x C x N (HWIO) filter reshaped; svdq_prepare_weights on Wm;
 *   Y      M x N row-major = the NHWC output batch x OH x OW x N.
 * Limits: KH, KW, stride in [1, 64], pad in [0, 64], KH <= H + 2 pad (and W),
 * batch*H*W*C and M below 2^31, K at most 2^25. Both formats: the INT4
 * entry points below, and their MXFP4 counterparts (the tiled layouts of the
 * MXFP4 section, prep by svdq_prepare_weights_mx on Wm).
 */

/* Host: out[k] (k < K) = max over the M patches of |patch matrix entry k|,
 * the calibration statistic of the convolution's smoothing factors. */
int svdq_conv_patch_absmax(const void* X, int x_dtype, int64_t batch, int64_t H, int64_t W,
                           int64_t C, int32_t KH, int32_t KW, int32_t stride, int32_t pad,
                           float* out);

/* Device: K1 on the patch matrix: a_codes (M x K/2), a_scales (M x K/64) and
 * D (M x R) as svdq_quantize_act_lowrank_down would give for the patch matrix
 * in memory (bit-exact). X 16-byte aligned. */
int svdq_quantize_act_lowrank_down_conv(const void* X, int x_dtype, int64_t batch, int64_t H,
                                        int64_t W, int64_t C, int32_t KH, int32_t KW,
                                        int32_t stride, int32_t pad, const float* inv_smooth,
                                        const uint16_t* L1p, int32_t R, uint8_t* a_codes,
                                        uint16_t* a_scales, float* D, hipStream_t stream);

/* Device: the whole convolution, K1 on the patch matrix into `ws`, then K2
 * (svdq_w4a4_gemm_lowrank_up) into Y (ldy = N). ws: 256-byte aligned, at
 * least svdq_linear_workspace_bytes(M, K, R, 64) bytes. */
int svdq_conv2d(const void* X, int x_dtype, int64_t batch, int64_t H, int64_t W, int64_t C,
                int32_t KH, int32_t KW, int32_t stride, int32_t pad, const float* inv_smooth,
                const uint16_t* L1p, const uint16_t* L2t, int32_t R, const uint8_t* w_codes,
                const uint16_t* w_scales, const float* bias, void* Y, int y_dtype, int64_t N,
                void* ws, size_t ws_bytes, int32_t activation, hipStream_t stream);

/* Device: K1 on the patch matrix writing the tiled INT4 layouts (a_ops_t,
 * a_scales_t, D_t), as svdq_quantize_act_lowrank_down_tiled would give for the
 * patch matrix in memory without a workspace (bit-exact). */
int svdq_quantize_act_lowrank_down_conv_tiled(const void* X, int x_dtype, int64_t batch,
                                              int64_t H, int64_t W, int64_t C, int32_t KH,
                                              int32_t KW, int32_t stride, int32_t pad,
                                              const float* inv_smooth, const uint16_t* L1p,
                                              int32_t R, uint8_t* a_ops_t, float* a_scales_t,
                                              uint16_t* D_t, hipStream_t stream);

/* Device: the whole convolution on the tiled INT4 path: K1 on the patch matrix
 * into `ws` in the tiled layouts, then K2T (svdq_w4a4_gemm_lowrank_up_tiled)
 * into Y (ldy = N); the weights tiled by svdq_pack_w4a4_tiles. ws: 256-byte
 * aligned, at least svdq_linear_tiled_workspace_bytes(M, K, R) bytes, and as
 * for svdq_linear_tiled svdq_gemm_tiled_workspace_bytes(M, N, K) more for the
 * split along K. */
int svdq_conv2d_tiled(const void* X, int x_dtype, int64_t batch, int64_t H, int64_t W, int64_t C,
                      int32_t KH, int32_t KW, int32_t stride, int32_t pad,
                      const float* inv_smooth, const uint16_t* L1p, const uint16_t* L2t,
                      int32_t R, const uint8_t* w_codes_t, const float* w_scales_t,
                      const float* bias, void* Y, int y_dtype, int64_t N, void* ws,
                      size_t ws_bytes, int32_t activation, hipStream_t stream);

/* Device: K1-MX on the patch matrix: the tiled E2M1 codes and E8M0 exponents
 * and D_t, as svdq_quantize_act_lowrank_down_mx would give for the patch
 * matrix in memory (bit-exact). */
int svdq_quantize_act_lowrank_down_conv_mx(const void* X, int x_dtype, int64_t batch, int64_t H,
                                           int64_t W, int64_t C, int32_t KH, int32_t KW,
                                           int32_t stride, int32_t pad, const float* inv_smooth,
                                           const uint16_t* L1p, int32_t R, uint8_t* a_codes_t,
                                           uint8_t* a_exps_t, uint16_t* D_t, hipStream_t stream);

/* Device: the whole convolution in MXFP4: K1-MX on the patch matrix into
 * `ws`, then K2-MX into Y (ldy = N). ws: 256-byte aligned, at least
 * svdq_linear_mx_workspace_bytes(M, K, R) bytes. */
int svdq_conv2d_mx(const void* X, int x_dtype, int64_t batch, int64_t H, int64_t W, int64_t C,
                   int32_t KH, int32_t KW, int32_t stride, int32_t pad, const float* inv_smooth,
                   const uint16_t* L1p, const uint16_t* L2t, int32_t R, const uint8_t* w_codes_t,
                   const uint8_t* w_exps_t, const float* bias, void* Y, int y_dtype, int64_t N,
                   void* ws, size_t ws_bytes, int32_t activation, hipStream_t stream);

/* Test hook: the exact integer partials P[m, n, g] for rows row0 .. row0+rows-1,
 * computed with the same operand unpacking and int8 matrix-core instruction
 * as K2. P: rows x N x (K/group) int32, row-major. 0 <= row0, row0+rows <= M. */
int svdq_debug_group_partials(const uint8_t* a_codes, const uint8_t* w_codes, int64_t M,
                              int64_t N, int64_t K, int32_t group, int64_t row0, int64_t rows,
                              int32_t* P, hipStream_t stream);

/* GELU, tanh form, between the two linears of a DiT MLP (not on the pages; the
 * textbook formula 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))), computed
 * in fp32 from fp16 and rounded to fp16. x and y may be the same buffer. */
int svdq_gelu_tanh_f16(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Measurement utilities (not part of the method): the shader clock during a
 * timed region. The pages give no hardware figures; the rooflines are priced
 * at the chip's peak clock, so a benchmark reports the clock it actually ran at.
 */

/* Host: the constant rate of the device's wall counter and the peak shader
 * clock, both in kHz (HIP device attributes of the current device). */
int svdq_clock_rates(int32_t* wall_khz, int32_t* peak_khz);

/* Device: one wave that, every `interval_ticks` ticks of the wall counter,
 * stores the pair (shader-clock cycle counter, wall counter) at
 * samples[1 + 2i], samples[2 + 2i], until *stop is nonzero (read with
 * agent-scope atomics) or max_samples pairs are stored; samples[0] = the
 * number stored. samples: device memory of 1 + 2*max_samples uint64 (8-byte
 * aligned); stop: device int32 (4-byte aligned), zero before the launch.
 * Limits: 1 <= max_samples <= 2^20, interval at most 10 ms and
 * max_samples * interval at most 60 s of wall ticks, so the wave always ends.
 * Launch it on a stream other than the timed one. */
int svdq_clock_probe(uint64_t* samples, int32_t max_samples, int64_t interval_ticks,
                     const int32_t* stop, hipStream_t stream);

/* Device: one wave that stores the wall counter at *stamp and, if stop is not
 * NULL, sets *stop = 1 (ending a running svdq_clock_probe). */
int svdq_clock_mark(uint64_t* stamp, int32_t* stop, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
