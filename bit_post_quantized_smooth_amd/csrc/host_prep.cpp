// Host-side offline preparation of an SVDQuant linear layer.
//
// chattools.cn overview, section "SVDQuant的技术原理" (technical principles):
// outliers are moved from the activations onto the weights by smoothing, the
// smoothed weight is split by SVD into a 16-bit low-rank branch and a residual,
// and the residual is quantized to 4 bits; the Eckart-Young-Mirsky item there
// is why the dominant singular values go to the branch. Section
// "SVDQuant的主要功能" (main features) adds LoRA integration without
// re-quantization. The SVDQuant abstract (ai-digest.ru) states the same steps.
//
// Built without floating-point contraction: the quantizer's fp32 divide and
// multiply must round exactly as the reading in svdq.h states.
#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <exception>
#include <new>
#include <vector>

#include "../../include/svdq.h"
#include "host_f16.hpp"
#include "host_internal.hpp"

namespace svdq {

namespace {
thread_local char g_last_error[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

void clear_error() { g_last_error[0] = '\0'; }

const char* last_error() { return g_last_error; }

// The 4-bit group quantizer on fp32 values (the reading in svdq.h):
// a = max|v|; s = fp16(min(a/7, 65504)); inv = s ? 1/s : 0;
// q = clamp(rint(v*inv), -7, 7). Writes `n/2` packed bytes and one scale.
static void quantize_group_f32(const float* v, int n, uint8_t* codes, uint16_t* scale) {
  float a = 0.0f;
  for (int i = 0; i < n; ++i) a = std::max(a, std::fabs(v[i]));
  volatile float s32 = a / 7.0f;                 // correctly rounded fp32 division
  float sc = std::min(static_cast<float>(s32), 65504.0f);
  const uint16_t s16 = f32_to_f16(sc);
  const float sf = f16_to_f32(s16);
  const float inv = (sf == 0.0f) ? 0.0f : 1.0f / sf;
  for (int i = 0; i < n; i += 2) {
    int q[2];
    for (int t = 0; t < 2; ++t) {
      volatile float prod = v[i + t] * inv;        // fp32 multiply, no contraction
      float r = std::nearbyint(static_cast<float>(prod));   // ties to even
      r = std::min(7.0f, std::max(-7.0f, r));
      q[t] = static_cast<int>(r);
    }
    codes[i / 2] = static_cast<uint8_t>((q[0] & 0xF) | ((q[1] & 0xF) << 4));
  }
  *scale = s16;
}

// The MXFP4 block quantizer on fp32 values (the reading in svdq.h): e is the
// exponent of the block's largest magnitude minus 2, at least -127 (the E8M0
// byte is the biased exponent field of max|v| minus 2, floored at 0); each
// value is v * 2^-e (exact in fp64) rounded to the nearest E2M1 value, ties to
// the even encoding, saturating at 6, sign bit kept. Writes 16 packed bytes
// and one E8M0 byte for 32 values.
static void quantize_block_mx(const float* v, uint8_t* codes, uint8_t* e8m0) {
  float a = 0.0f;
  for (int i = 0; i < SVDQ_MX_BLOCK; ++i) a = std::max(a, std::fabs(v[i]));
  uint32_t abits;
  std::memcpy(&abits, &a, sizeof(abits));
  const int e8 = std::max(static_cast<int>(abits >> 23) - 2, 0);
  // nearest E2M1 magnitude of m >= 0: counts the midpoints below m, a midpoint
  // itself going to the even code (E2M1 magnitudes 0 .5 1 1.5 2 3 4 6)
  auto code_of = [](double t) -> uint8_t {
    const double m = std::fabs(t);
    const int c = (m > 0.25) + (m >= 0.75) + (m > 1.25) + (m >= 1.75) + (m > 2.5) +
                  (m >= 3.5) + (m > 5.0);
    return static_cast<uint8_t>(c | (std::signbit(t) ? 8 : 0));
  };
  for (int i = 0; i < SVDQ_MX_BLOCK; i += 2) {
    const uint8_t c0 = code_of(std::ldexp(static_cast<double>(v[i]), 127 - e8));
    const uint8_t c1 = code_of(std::ldexp(static_cast<double>(v[i + 1]), 127 - e8));
    codes[i / 2] = static_cast<uint8_t>(c0 | (c1 << 4));
  }
  *e8m0 = static_cast<uint8_t>(e8);
}

int check_conv(int64_t batch, int64_t H, int64_t W, int64_t C, int32_t KH, int32_t KW,
               int32_t stride, int32_t pad, ConvShape& cs, const char* fn) {
  const int64_t lim = int64_t{1} << 31;
  if (batch < 1 || H < 1 || W < 1 || H >= lim || W >= lim || C < SVDQ_GROUP ||
      C % SVDQ_GROUP != 0 || KH < 1 || KH > 64 || KW < 1 || KW > 64 || stride < 1 ||
      stride > 64 || pad < 0 || pad > 64 || H + 2 * pad < KH || W + 2 * pad < KW) {
    set_error("%s: convolution batch=%lld H=%lld W=%lld C=%lld kernel %dx%d stride %d pad %d "
              "(need C a positive multiple of 64, kernel and stride in [1, 64], pad in [0, 64], "
              "kernel within the padded image)",
              fn, (long long)batch, (long long)H, (long long)W, (long long)C, KH, KW, stride, pad);
    return SVDQ_ERR_SHAPE;
  }
  cs.batch = batch; cs.H = H; cs.W = W; cs.C = C;
  cs.KH = KH; cs.KW = KW; cs.stride = stride; cs.pad = pad;
  cs.OH = (H + 2 * pad - KH) / stride + 1;
  cs.OW = (W + 2 * pad - KW) / stride + 1;
  cs.K = static_cast<int64_t>(KH) * KW * C;
  // element counts of the image and the number of output pixels, each below
  // 2^31 (checked factor by factor so the products cannot overflow)
  if (batch > lim / H || batch * H > lim / W || batch * H * W > (lim - 1) / C ||
      batch > lim / cs.OH || batch * cs.OH > (lim - 1) / cs.OW || cs.K > (int64_t{1} << 25)) {
    set_error("%s: image %lldx%lldx%lldx%lld or its %lld x %lld patch matrix too large", fn,
              (long long)batch, (long long)H, (long long)W, (long long)C,
              (long long)(batch * cs.OH * cs.OW), (long long)cs.K);
    return SVDQ_ERR_SHAPE;
  }
  cs.M = batch * cs.OH * cs.OW;
  return SVDQ_OK;
}

}  // namespace svdq

using namespace svdq;

#define SVDQ_TRY try {
#define SVDQ_CATCH                                               \
  }                                                              \
  catch (const std::bad_alloc&) {                                \
    set_error("host allocation failed");                         \
    return SVDQ_ERR_INTERNAL;                                    \
  }                                                              \
  catch (const std::exception& ex) {                             \
    set_error("internal error: %s", ex.what());                  \
    return SVDQ_ERR_INTERNAL;                                    \
  }                                                              \
  catch (...) {                                                  \
    set_error("internal error");                                 \
    return SVDQ_ERR_INTERNAL;                                    \
  }

namespace {

// The offline steps both 4-bit formats share: inv_smooth, the smoothing of W,
// the SVD split into the fp16 factors, and the fp32 residual R, handed column
// by column (K values down K for output column n) to quantize_column(col, n).
// Shapes and pointers are checked by the caller.
template <class QuantizeColumn>
int prepare_common(const char* fn, const float* W, const float* lambda, int64_t K, int64_t N,
                   int32_t rank, float* inv_smooth, uint16_t* L1t, uint16_t* L2t,
                   double* sigma, QuantizeColumn&& quantize_column) {
  const int64_t nmin = std::min(K, N);
  SVDQ_TRY
  // inv_smooth = 1/lambda in fp32; What = diag(lambda) W in fp64 (exact)
  for (int64_t k = 0; k < K; ++k) {
    volatile float inv = 1.0f / lambda[k];
    inv_smooth[k] = inv;
  }
  std::vector<double> What(static_cast<size_t>(K) * N);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < K; ++k) {
    const double l = static_cast<double>(lambda[k]);
    for (int64_t n = 0; n < N; ++n) What[k * N + n] = l * static_cast<double>(W[k * N + n]);
  }

  const bool need_svd = rank > 0 || sigma != nullptr;
  std::vector<double> L1(static_cast<size_t>(K) * rank, 0.0);   // fp16 values, K x r
  std::vector<double> L2(static_cast<size_t>(rank) * N, 0.0);   // fp16 values, r x N
  if (need_svd) {
    // Gram matrix of the shorter side, laid out so its rows are contiguous
    const bool rows_short = K <= N;     // B = What (K x N)  or  B = What^T (N x K)
    const int64_t n = nmin, m = rows_short ? N : K;
    std::vector<double> B;
    const double* Bp = What.data();
    if (!rows_short) {
      B.resize(static_cast<size_t>(N) * K);
#pragma omp parallel for schedule(static)
      for (int64_t i = 0; i < N; ++i)
        for (int64_t k = 0; k < K; ++k) B[i * K + k] = What[k * N + i];
      Bp = B.data();
    }
    std::vector<double> G(static_cast<size_t>(n) * n);
    gram_rows(Bp, n, m, G.data());
    std::vector<double> ev, Z, all;
    const int r = rank;
    if (!sym_top_eigen(G, n, r, ev, Z, sigma ? &all : nullptr)) {
      set_error("%s: eigen-solver did not converge", fn);
      return SVDQ_ERR_INTERNAL;
    }
    if (sigma)
      for (int64_t i = 0; i < n; ++i) sigma[i] = std::sqrt(std::max(0.0, all[i]));
    // Z (n x r): eigenvectors of B B^T = left singular vectors of B.
    // The other side is B^T z / s.  For rows_short, B = What: u = z, v = What^T u / s.
    // Otherwise B = What^T: v = z, u = What v / s.
    std::vector<double> s(r), u(static_cast<size_t>(K) * r), v(static_cast<size_t>(N) * r);
    for (int j = 0; j < r; ++j) s[j] = std::sqrt(std::max(0.0, ev[j]));
    std::vector<double>& zside = rows_short ? u : v;    // length n per column
    std::vector<double>& oside = rows_short ? v : u;    // length m per column
    for (int64_t i = 0; i < n; ++i)
      for (int j = 0; j < r; ++j) zside[i * r + j] = Z[i * r + j];
    // oside[:, j] = B^T z_j / s_j, B rows contiguous: accumulate row by row
    std::fill(oside.begin(), oside.end(), 0.0);
#pragma omp parallel
    {
      std::vector<double> acc(static_cast<size_t>(r));
#pragma omp for schedule(static)
      for (int64_t c = 0; c < m; ++c) {
        std::fill(acc.begin(), acc.end(), 0.0);
        for (int64_t i = 0; i < n; ++i) {
          const double b = Bp[i * m + c];
          const double* zr = Z.data() + i * r;
          for (int j = 0; j < r; ++j) acc[j] += b * zr[j];
        }
        for (int j = 0; j < r; ++j) oside[c * r + j] = s[j] > 1e-300 ? acc[j] / s[j] : 0.0;
      }
    }
    // canonical sign: the entry of largest magnitude of each u_j is positive
    for (int j = 0; j < r; ++j) {
      int64_t best = 0;
      double bmag = -1.0;
      for (int64_t k = 0; k < K; ++k) {
        const double a = std::fabs(u[k * r + j]);
        if (a > bmag) {
          bmag = a;
          best = k;
        }
      }
      if (u[best * r + j] < 0.0) {
        for (int64_t k = 0; k < K; ++k) u[k * r + j] = -u[k * r + j];
        for (int64_t c = 0; c < N; ++c) v[c * r + j] = -v[c * r + j];
      }
    }
    // L1 = fp16(U_r S^(1/2)), L2 = fp16(S^(1/2) V_r^T), each rounded once from fp64
    for (int j = 0; j < r; ++j) {
      const double h = std::sqrt(s[j]);
      for (int64_t k = 0; k < K; ++k) {
        const uint16_t q = f64_to_f16(u[k * r + j] * h);
        L1t[static_cast<int64_t>(j) * K + k] = q;
        L1[k * r + j] = f16_to_f64(q);
      }
      for (int64_t c = 0; c < N; ++c) {
        const uint16_t q = f64_to_f16(h * v[c * r + j]);
        L2t[c * r + j] = q;
        L2[static_cast<int64_t>(j) * N + c] = f16_to_f64(q);
      }
    }
  }

  // R = What - L1 L2 (from the stored fp16 factors; each product of two fp16
  // values is exact in fp64), rounded to fp32, then quantized down K for
  // each output column n.
  const int64_t NB = 16;   // columns per task
#pragma omp parallel
  {
    std::vector<float> col(static_cast<size_t>(NB) * K);
#pragma omp for schedule(dynamic, 1)
    for (int64_t n0 = 0; n0 < N; n0 += NB) {
      const int64_t nb = std::min(NB, N - n0);
      for (int64_t k = 0; k < K; ++k) {
        const double* wrow = &What[k * N + n0];
        const double* l1 = L1.data() + k * rank;
        for (int64_t c = 0; c < nb; ++c) {
          double acc = 0.0;
          for (int j = 0; j < rank; ++j) acc += l1[j] * L2[static_cast<int64_t>(j) * N + n0 + c];
          col[c * K + k] = static_cast<float>(wrow[c] - acc);
        }
      }
      for (int64_t c = 0; c < nb; ++c) quantize_column(&col[c * K], n0 + c);
    }
  }
  return SVDQ_OK;
  SVDQ_CATCH
}

// Checks shared by both prep functions.
int check_prep_args(const char* fn, int64_t K, int64_t N, int32_t rank) {
  if (K < SVDQ_GROUP || K % SVDQ_GROUP != 0) {
    set_error("%s: K=%lld (need K %% 64 == 0)", fn, (long long)K);
    return SVDQ_ERR_GROUP;
  }
  if (N < 1) {
    set_error("%s: N=%lld", fn, (long long)N);
    return SVDQ_ERR_SHAPE;
  }
  const int64_t nmin = std::min(K, N);
  if (rank < 0 || rank > nmin) {
    set_error("%s: rank %d outside [0, min(K,N)=%lld]", fn, rank, (long long)nmin);
    return SVDQ_ERR_RANK;
  }
  return SVDQ_OK;
}

}  // namespace

extern "C" {

int svdq_channel_absmax(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                        float* out) {
  clear_error();
  if (!X || !out) {
    set_error("svdq_channel_absmax: null pointer");
    return SVDQ_ERR_NULL;
  }
  if (x_dtype != SVDQ_F16 && x_dtype != SVDQ_F32) {
    set_error("svdq_channel_absmax: x_dtype %d", x_dtype);
    return SVDQ_ERR_DTYPE;
  }
  if (M < 1 || K < 1 || ldx < K) {
    set_error("svdq_channel_absmax: bad shape M=%lld K=%lld ldx=%lld", (long long)M,
              (long long)K, (long long)ldx);
    return SVDQ_ERR_SHAPE;
  }
  SVDQ_TRY
  const int nt = omp_get_max_threads();
  std::vector<float> part(static_cast<size_t>(nt) * K, 0.0f);
#pragma omp parallel
  {
    float* mine = &part[static_cast<size_t>(omp_get_thread_num()) * K];
#pragma omp for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
      if (x_dtype == SVDQ_F32) {
        const float* row = static_cast<const float*>(X) + m * ldx;
        for (int64_t k = 0; k < K; ++k) mine[k] = std::max(mine[k], std::fabs(row[k]));
      } else {
        const uint16_t* row = static_cast<const uint16_t*>(X) + m * ldx;
        for (int64_t k = 0; k < K; ++k) mine[k] = std::max(mine[k], std::fabs(f16_to_f32(row[k])));
      }
    }
  }
  for (int64_t k = 0; k < K; ++k) {
    float a = 0.0f;
    for (int t = 0; t < nt; ++t) a = std::max(a, part[static_cast<size_t>(t) * K + k]);
    out[k] = a;
  }
  return SVDQ_OK;
  SVDQ_CATCH
}

int svdq_conv_patch_absmax(const void* X, int x_dtype, int64_t batch, int64_t H, int64_t W,
                           int64_t C, int32_t KH, int32_t KW, int32_t stride, int32_t pad,
                           float* out) {
  clear_error();
  const char* fn = "svdq_conv_patch_absmax";
  if (!X || !out) {
    set_error("%s: null pointer", fn);
    return SVDQ_ERR_NULL;
  }
  if (x_dtype != SVDQ_F16 && x_dtype != SVDQ_F32) {
    set_error("%s: x_dtype %d", fn, x_dtype);
    return SVDQ_ERR_DTYPE;
  }
  ConvShape cs;
  if (int s = check_conv(batch, H, W, C, KH, KW, stride, pad, cs, fn)) return s;
  SVDQ_TRY
  // column (kh, kw, c) of the patch matrix holds pixel (oh*stride + kh - pad,
  // ow*stride + kw - pad) of every image, or 0 outside it (which never raises
  // a maximum of magnitudes)
  const int64_t taps = static_cast<int64_t>(KH) * KW;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < taps; ++t) {
    const int64_t kh = t / KW, kw = t % KW;
    float* o = out + t * C;
    for (int64_t c = 0; c < C; ++c) o[c] = 0.0f;
    for (int64_t b = 0; b < batch; ++b)
      for (int64_t oh = 0; oh < cs.OH; ++oh) {
        const int64_t ih = oh * stride + kh - pad;
        if (ih < 0 || ih >= H) continue;
        for (int64_t ow = 0; ow < cs.OW; ++ow) {
          const int64_t iw = ow * stride + kw - pad;
          if (iw < 0 || iw >= W) continue;
          const int64_t px = ((b * H + ih) * W + iw) * C;
          if (x_dtype == SVDQ_F32) {
            const float* row = static_cast<const float*>(X) + px;
            for (int64_t c = 0; c < C; ++c) o[c] = std::max(o[c], std::fabs(row[c]));
          } else {
            const uint16_t* row = static_cast<const uint16_t*>(X) + px;
            for (int64_t c = 0; c < C; ++c) o[c] = std::max(o[c], std::fabs(f16_to_f32(row[c])));
          }
        }
      }
  }
  return SVDQ_OK;
  SVDQ_CATCH
}

int svdq_smoothing_factors(const float* x_absmax, const float* W, int64_t K, int64_t N,
                           float* lambda) {
  clear_error();
  if (!x_absmax || !W || !lambda) {
    set_error("svdq_smoothing_factors: null pointer");
    return SVDQ_ERR_NULL;
  }
  if (K < 1 || N < 1) {
    set_error("svdq_smoothing_factors: bad shape K=%lld N=%lld", (long long)K, (long long)N);
    return SVDQ_ERR_SHAPE;
  }
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < K; ++j) {
    double wa = 0.0;
    const float* row = W + j * N;
    for (int64_t n = 0; n < N; ++n) wa = std::max(wa, std::fabs(static_cast<double>(row[n])));
    const double xa = std::fabs(static_cast<double>(x_absmax[j]));
    double lam = 1.0;
    if (xa > 0.0 && wa > 0.0) lam = std::sqrt(xa / wa);
    lambda[j] = static_cast<float>(lam);
  }
  return SVDQ_OK;
}

int svdq_prepare_weights(const float* W, const float* lambda, int64_t K, int64_t N, int32_t rank,
                         int32_t group, float* inv_smooth, uint16_t* L1t, uint16_t* L2t,
                         uint8_t* w_codes, uint16_t* w_scales, double* sigma) {
  clear_error();
  if (!W || !lambda || !inv_smooth || !w_codes || !w_scales || (rank > 0 && (!L1t || !L2t))) {
    set_error("svdq_prepare_weights: null pointer");
    return SVDQ_ERR_NULL;
  }
  if (group != SVDQ_GROUP) {
    set_error("svdq_prepare_weights: group=%d (need 64)", group);
    return SVDQ_ERR_GROUP;
  }
  const int st = check_prep_args("svdq_prepare_weights", K, N, rank);
  if (st != SVDQ_OK) return st;
  const int64_t G = K / SVDQ_GROUP;
  return prepare_common("svdq_prepare_weights", W, lambda, K, N, rank, inv_smooth, L1t, L2t,
                        sigma, [&](const float* col, int64_t n) {
                          for (int64_t g = 0; g < G; ++g)
                            quantize_group_f32(col + g * SVDQ_GROUP, SVDQ_GROUP,
                                               &w_codes[n * (K / 2) + g * (SVDQ_GROUP / 2)],
                                               &w_scales[n * G + g]);
                        });
}

int svdq_prepare_weights_mx(const float* W, const float* lambda, int64_t K, int64_t N,
                            int32_t rank, float* inv_smooth, uint16_t* L1t, uint16_t* L2t,
                            uint8_t* w_codes, uint8_t* w_e8m0, double* sigma) {
  clear_error();
  if (!W || !lambda || !inv_smooth || !w_codes || !w_e8m0 || (rank > 0 && (!L1t || !L2t))) {
    set_error("svdq_prepare_weights_mx: null pointer");
    return SVDQ_ERR_NULL;
  }
  const int st = check_prep_args("svdq_prepare_weights_mx", K, N, rank);
  if (st != SVDQ_OK) return st;
  const int64_t NBK = K / SVDQ_MX_BLOCK;
  return prepare_common("svdq_prepare_weights_mx", W, lambda, K, N, rank, inv_smooth, L1t, L2t,
                        sigma, [&](const float* col, int64_t n) {
                          for (int64_t b = 0; b < NBK; ++b)
                            quantize_block_mx(col + b * SVDQ_MX_BLOCK,
                                              &w_codes[n * (K / 2) + b * (SVDQ_MX_BLOCK / 2)],
                                              &w_e8m0[n * NBK + b]);
                        });
}

size_t svdq_mx_codes_tiled_bytes(int64_t rows, int64_t K) {
  if (rows < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0) return 0;
  return static_cast<size_t>((rows + 15) / 16) * static_cast<size_t>((K + 127) / 128) * 1024;
}

size_t svdq_mx_exps_tiled_bytes(int64_t rows, int64_t K) {
  if (rows < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0) return 0;
  return static_cast<size_t>((rows + 63) / 64) * static_cast<size_t>((K + 127) / 128) * 256;
}

int svdq_pack_mx_tiles(const uint8_t* codes, const uint8_t* e8m0, int64_t rows, int64_t K,
                       uint8_t* codes_t, uint8_t* exps_t) {
  clear_error();
  if (!codes || !e8m0 || !codes_t || !exps_t) {
    set_error("svdq_pack_mx_tiles: null pointer");
    return SVDQ_ERR_NULL;
  }
  if (K < SVDQ_GROUP || K % SVDQ_GROUP != 0) {
    set_error("svdq_pack_mx_tiles: K=%lld (need K %% 64 == 0)", (long long)K);
    return SVDQ_ERR_GROUP;
  }
  if (rows < 1) {
    set_error("svdq_pack_mx_tiles: rows=%lld", (long long)rows);
    return SVDQ_ERR_SHAPE;
  }
  const int64_t C = (K + 127) / 128, kb = K / 2, ks = K / SVDQ_MX_BLOCK;
  const int64_t nb = (rows + 15) / 16, ng = (rows + 63) / 64;
  // codes: block (b, c), lane l = 16q + r: row 16b + r, bytes 64c + 16q .. +15
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b)
    for (int64_t c = 0; c < C; ++c)
      for (int l = 0; l < 64; ++l) {
        const int64_t row = 16 * b + (l & 15), off = 64 * c + 16 * (l >> 4);
        uint8_t* dst = codes_t + ((b * C + c) * 64 + l) * 16;
        if (row < rows && off < kb)
          std::memcpy(dst, codes + row * kb + off, 16);
        else
          std::memset(dst, 0, 16);
      }
  // exponents: block (g, c), byte 4l + i: row 64g + 16i + r, 32-block 4c + q
#pragma omp parallel for schedule(static)
  for (int64_t g = 0; g < ng; ++g)
    for (int64_t c = 0; c < C; ++c)
      for (int l = 0; l < 64; ++l)
        for (int i = 0; i < 4; ++i) {
          const int64_t row = 64 * g + 16 * i + (l & 15), blk = 4 * c + (l >> 4);
          exps_t[((g * C + c) * 64 + l) * 4 + i] =
              (row < rows && blk < ks) ? e8m0[row * ks + blk] : uint8_t{127};
        }
  return SVDQ_OK;
}

int svdq_prepare_weights_w4a16(const float* W, int64_t K, int64_t N, uint8_t* w_codes,
                               uint16_t* w_scales) {
  clear_error();
  if (!W || !w_codes || !w_scales) {
    set_error("svdq_prepare_weights_w4a16: null pointer");
    return SVDQ_ERR_NULL;
  }
  const int st = check_prep_args("svdq_prepare_weights_w4a16", K, N, 0);
  if (st != SVDQ_OK) return st;
  SVDQ_TRY
  const int64_t G = K / SVDQ_GROUP;
#pragma omp parallel
  {
    std::vector<float> col(static_cast<size_t>(K));
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      for (int64_t k = 0; k < K; ++k) col[k] = W[k * N + n];
      for (int64_t g = 0; g < G; ++g)
        quantize_group_f32(&col[g * SVDQ_GROUP], SVDQ_GROUP,
                           &w_codes[n * (K / 2) + g * (SVDQ_GROUP / 2)], &w_scales[n * G + g]);
    }
  }
  return SVDQ_OK;
  SVDQ_CATCH
}

size_t svdq_w4a16_codes_tiled_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0) return 0;
  return static_cast<size_t>((N + 15) / 16) * static_cast<size_t>(K / 32) * 256;
}

size_t svdq_w4a16_scales_tiled_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0) return 0;
  return static_cast<size_t>((N + 63) / 64) * static_cast<size_t>(K / SVDQ_GROUP) * 128;
}

int svdq_pack_w4a16_tiles(const uint8_t* w_codes, const uint16_t* w_scales, int64_t N, int64_t K,
                          uint8_t* codes_t, uint16_t* scales_t) {
  clear_error();
  if (!w_codes || !w_scales || !codes_t || !scales_t) {
    set_error("svdq_pack_w4a16_tiles: null pointer");
    return SVDQ_ERR_NULL;
  }
  if (K < SVDQ_GROUP || K % SVDQ_GROUP != 0) {
    set_error("svdq_pack_w4a16_tiles: K=%lld (need K %% 64 == 0)", (long long)K);
    return SVDQ_ERR_GROUP;
  }
  if (N < 1) {
    set_error("svdq_pack_w4a16_tiles: N=%lld", (long long)N);
    return SVDQ_ERR_SHAPE;
  }
  const int64_t S = K / 32, G = K / SVDQ_GROUP, kb = K / 2;
  const int64_t nb = (N + 15) / 16, ng = (N + 63) / 64;
  // codes: block (b, s), lane l = 16q + r: column 16b + r, bytes 16s + 4q .. +3,
  // each nibble with bit 3 flipped (code + 8)
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b)
    for (int64_t s = 0; s < S; ++s)
      for (int l = 0; l < 64; ++l) {
        const int64_t n = 16 * b + (l & 15);
        uint8_t* dst = codes_t + ((b * S + s) * 64 + l) * 4;
        for (int j = 0; j < 4; ++j)
          dst[j] = n < N ? static_cast<uint8_t>(w_codes[n * kb + 16 * s + 4 * (l >> 4) + j] ^ 0x88u)
                         : uint8_t{0x88};
      }
  // scales: block (c, g), entry 4r + j: column 64c + 16j + r, group g (0 past N)
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < ng; ++c)
    for (int64_t g = 0; g < G; ++g)
      for (int r = 0; r < 16; ++r)
        for (int j = 0; j < 4; ++j) {
          const int64_t n = 64 * c + 16 * j + r;
          scales_t[(c * G + g) * 64 + 4 * r + j] = n < N ? w_scales[n * G + g] : uint16_t{0};
        }
  return SVDQ_OK;
}

size_t svdq_int4_act_tiled_bytes(int64_t M, int64_t K) {
  if (M < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0) return 0;
  return static_cast<size_t>((M + 15) / 16) * static_cast<size_t>(K / SVDQ_GROUP) * 1024;
}

size_t svdq_int4_act_scales_tiled_bytes(int64_t M, int64_t K) {
  if (M < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0) return 0;
  return static_cast<size_t>((M + 127) / 128) * static_cast<size_t>(K / SVDQ_GROUP) * 512;
}

size_t svdq_int4_d_tiled_bytes(int64_t M, int32_t R) {
  if (M < 1 || R < 1) return 0;
  return static_cast<size_t>((M + 15) / 16) * static_cast<size_t>((R + 31) / 32) * 1024;
}

size_t svdq_int4_w_codes_tiled_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0) return 0;
  return static_cast<size_t>((N + 31) / 32) * static_cast<size_t>(K / SVDQ_GROUP) * 1024;
}

size_t svdq_int4_w_scales_tiled_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0) return 0;
  return static_cast<size_t>((N + 31) / 32) * static_cast<size_t>(K / SVDQ_GROUP) * 256;
}

int svdq_pack_w4a4_tiles(const uint8_t* w_codes, const uint16_t* w_scales, int64_t N, int64_t K,
                         uint8_t* w_codes_t, float* w_scales_t) {
  clear_error();
  if (!w_codes || !w_scales || !w_codes_t || !w_scales_t) {
    set_error("svdq_pack_w4a4_tiles: null pointer");
    return SVDQ_ERR_NULL;
  }
  if (K < SVDQ_GROUP || K % SVDQ_GROUP != 0) {
    set_error("svdq_pack_w4a4_tiles: K=%lld (need K %% 64 == 0)", (long long)K);
    return SVDQ_ERR_GROUP;
  }
  if (N < 1) {
    set_error("svdq_pack_w4a4_tiles: N=%lld", (long long)N);
    return SVDQ_ERR_SHAPE;
  }
  const int64_t G = K / SVDQ_GROUP, kb = K / 2, ns = (N + 31) / 32;
  // codes: block (s, g), lane l = 16q + r: bytes 0..7 = codes of column
  // 32s + r, bytes 8..15 = codes of column 32s + 16 + r, each the 8 bytes
  // 32g + 8q .. +7 of the column's row (0 past N)
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < ns; ++s)
    for (int64_t g = 0; g < G; ++g)
      for (int l = 0; l < 64; ++l)
        for (int j = 0; j < 2; ++j) {
          const int64_t n = 32 * s + 16 * j + (l & 15);
          uint8_t* dst = w_codes_t + ((s * G + g) * 64 + l) * 16 + 8 * j;
          for (int t = 0; t < 8; ++t)
            dst[t] = n < N ? w_codes[n * kb + 32 * g + 8 * (l >> 4) + t] : uint8_t{0};
        }
  // scales: block (s, g), entries 16q + 8j + 2e and +1: the pair
  // (s/256, -12582912 s/256) of column 32s + 16j + 4q + e (0 past N); both
  // products are exact in fp32 (a power of two; 12582912/256 = 3 * 2^14 adds
  // two bits to the 11 of an fp16 significand)
#pragma omp parallel for schedule(static)
  for (int64_t s = 0; s < ns; ++s)
    for (int64_t g = 0; g < G; ++g)
      for (int q = 0; q < 4; ++q)
        for (int j = 0; j < 2; ++j)
          for (int e = 0; e < 4; ++e) {
            const int64_t n = 32 * s + 16 * j + 4 * q + e;
            const float sw = n < N ? f16_to_f32(w_scales[n * G + g]) : 0.f;
            float* dst = w_scales_t + (s * G + g) * 64 + 16 * q + 8 * j + 2 * e;
            dst[0] = sw * 0.00390625f;
            dst[1] = sw * -49152.0f;
          }
  return SVDQ_OK;
}

int svdq_concat_lora(const uint16_t* L1t, const uint16_t* L2t, int64_t K, int64_t N, int32_t rank,
                     const float* lambda, const uint16_t* A, const uint16_t* B, int32_t rl,
                     float scale, uint16_t* L1t_out, uint16_t* L2t_out) {
  clear_error();
  if (!lambda || !A || !B || !L1t_out || !L2t_out || (rank > 0 && (!L1t || !L2t))) {
    set_error("svdq_concat_lora: null pointer");
    return SVDQ_ERR_NULL;
  }
  if (K < 1 || N < 1) {
    set_error("svdq_concat_lora: bad shape");
    return SVDQ_ERR_SHAPE;
  }
  if (rank < 0 || rl < 1) {
    set_error("svdq_concat_lora: rank=%d rl=%d", rank, rl);
    return SVDQ_ERR_RANK;
  }
  const int64_t ro = static_cast<int64_t>(rank) + rl;
  // L1' rows 0..rank-1 are L1; rows rank.. are fp16(lambda (.) A * scale), transposed
  if (rank > 0) std::memcpy(L1t_out, L1t, sizeof(uint16_t) * static_cast<size_t>(rank) * K);
  const double sc = static_cast<double>(scale);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < K; ++k) {
    const double l = static_cast<double>(lambda[k]);
    for (int32_t j = 0; j < rl; ++j) {
      double t = l * f16_to_f64(A[k * rl + j]);   // exact
      t = t * sc;                                   // one fp64 rounding
      L1t_out[(rank + j) * K + k] = f64_to_f16(t);
    }
  }
  // L2' = [L2 ; B], stored transposed: row n = [L2t[n, :], B[:, n]]
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int32_t j = 0; j < rank; ++j) L2t_out[n * ro + j] = L2t[n * rank + j];
    for (int32_t j = 0; j < rl; ++j) L2t_out[n * ro + rank + j] = B[static_cast<int64_t>(j) * N + n];
  }
  return SVDQ_OK;
}

int svdq_pack_lowrank_down(const uint16_t* L1t, int64_t K, int32_t R, uint16_t* L1p) {
  clear_error();
  if (!L1t || !L1p) {
    set_error("svdq_pack_lowrank_down: null pointer");
    return SVDQ_ERR_NULL;
  }
  if (K < SVDQ_GROUP || K % SVDQ_GROUP != 0) {
    set_error("svdq_pack_lowrank_down: K=%lld is not a positive multiple of %d", (long long)K,
              SVDQ_GROUP);
    return SVDQ_ERR_GROUP;
  }
  if (R < 16 || R % 16 != 0 || R > SVDQ_MAX_RANK) {
    set_error("svdq_pack_lowrank_down: R=%d", R);
    return SVDQ_ERR_RANK;
  }
  // operand (g, c, h), lane = q*16 + rl, element j  <-  L1t[c*16 + rl][g*64 + q*16 + h*8 + j]
  const int64_t G = K / SVDQ_GROUP, ncb = R / 16;
#pragma omp parallel for schedule(static)
  for (int64_t g = 0; g < G; ++g)
    for (int64_t c = 0; c < ncb; ++c)
      for (int h = 0; h < 2; ++h)
        for (int lane = 0; lane < 64; ++lane) {
          const int rl = lane & 15, q = lane >> 4;
          const uint16_t* src = L1t + (c * 16 + rl) * K + g * SVDQ_GROUP + q * 16 + h * 8;
          uint16_t* dst = L1p + (((g * ncb + c) * 2 + h) * 64 + lane) * 8;
          for (int j = 0; j < 8; ++j) dst[j] = src[j];
        }
  return SVDQ_OK;
}

int svdq_pack_lowrank(const uint16_t* L1, const uint16_t* L2, int64_t K, int64_t N, int32_t R,
                      uint16_t* L1p, uint16_t* L2t) {
  clear_error();
  if (!L1 || !L2 || !L1p || !L2t) {
    set_error("svdq_pack_lowrank: null pointer");
    return SVDQ_ERR_NULL;
  }
  if (K < SVDQ_GROUP || K % SVDQ_GROUP != 0) {
    set_error("svdq_pack_lowrank: K=%lld is not a positive multiple of %d", (long long)K,
              SVDQ_GROUP);
    return SVDQ_ERR_GROUP;
  }
  if (N < 1) {
    set_error("svdq_pack_lowrank: N=%lld", (long long)N);
    return SVDQ_ERR_SHAPE;
  }
  if (R < 16 || R % 16 != 0 || R > SVDQ_MAX_RANK) {
    set_error("svdq_pack_lowrank: R=%d", R);
    return SVDQ_ERR_RANK;
  }
  // operand (g, c, h), lane = q*16 + rl, element j  <-  L1[g*64 + q*16 + h*8 + j][c*16 + rl]
  const int64_t G = K / SVDQ_GROUP, ncb = R / 16;
#pragma omp parallel for schedule(static)
  for (int64_t g = 0; g < G; ++g)
    for (int64_t c = 0; c < ncb; ++c)
      for (int h = 0; h < 2; ++h)
        for (int lane = 0; lane < 64; ++lane) {
          const int rl = lane & 15, q = lane >> 4;
          const int64_t k0 = g * SVDQ_GROUP + q * 16 + h * 8, r = c * 16 + rl;
          uint16_t* dst = L1p + (((g * ncb + c) * 2 + h) * 64 + lane) * 8;
          for (int j = 0; j < 8; ++j) dst[j] = L1[(k0 + j) * R + r];
        }
  // L2t[n][r] = L2[r][n]
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int32_t r = 0; r < R; ++r) L2t[n * R + r] = L2[static_cast<int64_t>(r) * N + n];
  return SVDQ_OK;
}

int svdq_abi_version(void) { return SVDQ_ABI_VERSION; }

const char* svdq_status_str(int status) {
  switch (status) {
    case SVDQ_OK: return "ok";
    case SVDQ_ERR_NULL: return "null pointer";
    case SVDQ_ERR_SHAPE: return "bad shape or stride";
    case SVDQ_ERR_ALIGN: return "misaligned pointer or stride";
    case SVDQ_ERR_DTYPE: return "unknown dtype";
    case SVDQ_ERR_RANK: return "bad rank";
    case SVDQ_ERR_WORKSPACE: return "workspace too small";
    case SVDQ_ERR_HIP: return "HIP error";
    case SVDQ_ERR_NO_DEVICE: return "no usable GPU";
    case SVDQ_ERR_INTERNAL: return "internal error";
    case SVDQ_ERR_GROUP: return "unsupported group size";
    case SVDQ_ERR_ACT: return "unknown activation";
    default: return "unknown status";
  }
}

const char* svdq_last_error(void) { return svdq::last_error(); }

}  // extern "C"
