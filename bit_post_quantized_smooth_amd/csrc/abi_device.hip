// C ABI of the device entry points: argument checks, workspace carving and
// kernel launches. Every check runs on the host before anything is enqueued;
// on an error nothing is launched or written.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/svdq.h"
#include "device_launch.hpp"
#include "host_internal.hpp"

using namespace svdq;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int device_ready() {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    set_error("no usable GPU: %s", hipGetErrorString(e));
    return SVDQ_ERR_NO_DEVICE;
  }
  return SVDQ_OK;
}

int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return SVDQ_ERR_HIP;
  }
  return SVDQ_OK;
}

int esize(int dtype) { return dtype == SVDQ_F16 ? 2 : 4; }

bool known_dtype(int d) { return d == SVDQ_F16 || d == SVDQ_F32; }

int check_common(int64_t M, int64_t K, int32_t R, int32_t group, const char* fn) {
  if (group != SVDQ_GROUP || K < SVDQ_GROUP || K % SVDQ_GROUP != 0) {
    set_error("%s: group=%d K=%lld (need group 64 and K a positive multiple of 64)", fn, group,
              (long long)K);
    return SVDQ_ERR_GROUP;
  }
  if (M < 1 || M > (int64_t(1) << 31) * 16 - 16) {
    set_error("%s: M=%lld out of range", fn, (long long)M);
    return SVDQ_ERR_SHAPE;
  }
  if (R < 0 || R > SVDQ_MAX_RANK || R % 16 != 0) {
    set_error("%s: R=%d (need 0 <= R <= %d, R %% 16 == 0)", fn, R, SVDQ_MAX_RANK);
    return SVDQ_ERR_RANK;
  }
  return SVDQ_OK;
}

// Longest X row (elements) the pre-kernel accepts: 16 rows of fp32 stay below
// 2^31 bytes, so per-lane offsets fit in 32 bits.
constexpr int64_t kMaxRowElems = int64_t{1} << 25;

// a_meta: the fp16 scales, or the E8M0 exponents of the MXFP4 entry points
int validate_k1(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                const float* inv_smooth, const uint16_t* L1p, int32_t R, int32_t group,
                const uint8_t* a_codes, const void* a_scales, const float* D, const char* fn) {
  if (!X || !inv_smooth || !a_codes || !a_scales || (R > 0 && (!L1p || !D))) {
    set_error("%s: null pointer", fn);
    return SVDQ_ERR_NULL;
  }
  if (!known_dtype(x_dtype)) {
    set_error("%s: x_dtype %d", fn, x_dtype);
    return SVDQ_ERR_DTYPE;
  }
  if (int s = check_common(M, K, R, group, fn)) return s;
  if (ldx < K) {
    set_error("%s: ldx=%lld < K=%lld", fn, (long long)ldx, (long long)K);
    return SVDQ_ERR_SHAPE;
  }
  // the kernel addresses 16 rows of X with 32-bit offsets
  if (ldx > kMaxRowElems) {
    set_error("%s: ldx=%lld exceeds %lld", fn, (long long)ldx, (long long)kMaxRowElems);
    return SVDQ_ERR_SHAPE;
  }
  if (!aligned16(X) || !aligned16(inv_smooth) || !aligned16(a_codes) || !aligned16(a_scales) ||
      (R > 0 && (!aligned16(L1p) || !aligned16(D))) || (ldx * esize(x_dtype)) % 16 != 0) {
    set_error("%s: device pointers and the X row stride must be 16-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  return SVDQ_OK;
}

int check_activation(int32_t activation, const char* fn) {
  if (activation != SVDQ_ACT_NONE && activation != SVDQ_ACT_GELU_TANH) {
    set_error("%s: activation %d", fn, activation);
    return SVDQ_ERR_ACT;
  }
  return SVDQ_OK;
}

int validate_k2(const uint8_t* a_codes, const void* a_scales, const uint8_t* w_codes,
                const void* w_scales, const float* D, const uint16_t* L2t, int32_t R,
                const float* bias, const void* Y, int y_dtype, int64_t M, int64_t N, int64_t K,
                int64_t ldy, int32_t group, const char* fn) {
  if (!a_codes || !a_scales || !w_codes || !w_scales || !Y || (R > 0 && (!D || !L2t))) {
    set_error("%s: null pointer", fn);
    return SVDQ_ERR_NULL;
  }
  if (!known_dtype(y_dtype)) {
    set_error("%s: y_dtype %d", fn, y_dtype);
    return SVDQ_ERR_DTYPE;
  }
  if (int s = check_common(M, K, R, group, fn)) return s;
  if (N < 1 || ldy < N || ((M + 127) / 128) * ((N + 127) / 128) > 0x7FFFFFFF) {
    set_error("%s: N=%lld ldy=%lld", fn, (long long)N, (long long)ldy);
    return SVDQ_ERR_SHAPE;
  }
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      (R > 0 && (!aligned16(D) || !aligned16(L2t)))) {
    set_error("%s: codes, scales or exponents, D and L2t must be 16-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  if ((reinterpret_cast<uintptr_t>(Y) % esize(y_dtype)) != 0 ||
      (bias && (reinterpret_cast<uintptr_t>(bias) & 3u) != 0)) {
    set_error("%s: Y and bias must be aligned to their element size", fn);
    return SVDQ_ERR_ALIGN;
  }
  return SVDQ_OK;
}

struct WsLayout {
  size_t codes, scales, d, part, total;
};

// The split pre-kernel's partial D tiles (k1_split_bytes; 0 when the shape is
// not split on this device).
size_t part_bytes(int64_t M, int64_t K, int32_t R, int fmt) {
  return round_up(k1_split_bytes(M, K, R, fmt, false), 256);
}

// INT4: codes M x K/2, fp16 scales M x K/64; MXFP4: the tiled codes and
// exponents (ceil(M/16) and ceil(M/64) blocks of 1024 and 256 bytes per chunk
// of 128 along K)
WsLayout ws_layout(int64_t M, int64_t K, int32_t R, bool mx) {
  WsLayout w;
  w.codes = 0;
  if (mx) {
    const size_t C = static_cast<size_t>((K + 127) / 128);
    w.scales = round_up(static_cast<size_t>((M + 15) / 16) * C * 1024, 256);
    w.d = w.scales + round_up(static_cast<size_t>((M + 63) / 64) * C * 256, 256);
  } else {
    w.scales = round_up(static_cast<size_t>(M) * (K / 2), 256);
    w.d = w.scales + round_up(static_cast<size_t>(M) * (K / SVDQ_GROUP) * 2, 256);
  }
  // D: fp32 M x R, or for MXFP4 fp16 in operand order (ceil(M/16) x
  // ceil(R/32) blocks of 1 KB); MXFP4 then the split pre-kernel's partials
  w.part = w.d + (mx ? round_up(static_cast<size_t>((M + 15) / 16) * ((R + 31) / 32) * 1024, 256)
                     : round_up(static_cast<size_t>(M) * R * 4, 256));
  w.total = w.part + (mx ? part_bytes(M, K, R, kK1Mx) : 0);
  return w;
}

// The tiled INT4 path: operand blocks ceil(M/16) x K/64 of 1 KB, scales
// ceil(M/128) x K/64 of 512 bytes, fp16 D in operand order ceil(M/16) x
// ceil(R/32) blocks of 1 KB, then the split pre-kernel's partials.
WsLayout tiled_ws_layout(int64_t M, int64_t K, int32_t R) {
  WsLayout w;
  const size_t G = static_cast<size_t>(K / SVDQ_GROUP);
  w.codes = 0;
  w.scales = round_up(static_cast<size_t>((M + 15) / 16) * G * 1024, 256);
  w.d = w.scales + round_up(static_cast<size_t>((M + 127) / 128) * G * 512, 256);
  w.part = w.d + round_up(static_cast<size_t>((M + 15) / 16) * ((R + 31) / 32) * 1024, 256);
  w.total = w.part + part_bytes(M, K, R, kK1Int4Tiled);
  return w;
}

ConvGeom conv_geom(const ConvShape& cs) {
  return ConvGeom{static_cast<int32_t>(cs.H), static_cast<int32_t>(cs.W),
                  static_cast<int32_t>(cs.C), cs.KH, cs.KW, cs.stride, cs.pad,
                  static_cast<int32_t>(cs.OH), static_cast<int32_t>(cs.OW)};
}

}  // namespace

extern "C" {

int svdq_quantize_act_lowrank_down(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                                   const float* inv_smooth, const uint16_t* L1p, int32_t R,
                                   int32_t group, uint8_t* a_codes, uint16_t* a_scales, float* D,
                                   hipStream_t stream) {
  clear_error();
  if (int s = validate_k1(X, x_dtype, M, K, ldx, inv_smooth, L1p, R, group, a_codes, a_scales, D,
                          "svdq_quantize_act_lowrank_down"))
    return s;
  if (int s = device_ready()) return s;
  return check_hip(launch_k1(X, x_dtype == SVDQ_F16, M, K, ldx, inv_smooth, L1p, R, a_codes,
                             a_scales, false, D, stream),
                   "svdq_quantize_act_lowrank_down launch");
}

int svdq_w4a4_gemm_lowrank_up(const uint8_t* a_codes, const uint16_t* a_scales,
                              const uint8_t* w_codes, const uint16_t* w_scales, const float* D,
                              const uint16_t* L2t, int32_t R, const float* bias, void* Y,
                              int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy,
                              int32_t group, int32_t activation, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_w4a4_gemm_lowrank_up";
  if (int s = validate_k2(a_codes, a_scales, w_codes, w_scales, D, L2t, R, bias, Y, y_dtype, M, N,
                          K, ldy, group, fn))
    return s;
  if (int s = check_activation(activation, fn)) return s;
  if (int s = device_ready()) return s;
  return check_hip(launch_k2(a_codes, a_scales, w_codes, w_scales, D, L2t, R, bias, Y,
                             y_dtype == SVDQ_F16, M, N, K, ldy, activation == SVDQ_ACT_GELU_TANH, stream),
                   "svdq_w4a4_gemm_lowrank_up launch");
}

size_t svdq_linear_workspace_bytes(int64_t M, int64_t K, int32_t R, int32_t group) {
  if (M < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0 || group != SVDQ_GROUP || R < 0) return 0;
  return ws_layout(M, K, R, false).total;
}

int svdq_linear(const void* X, int x_dtype, int64_t ldx, const float* inv_smooth,
                const uint16_t* L1p, const uint16_t* L2t, int32_t R, const uint8_t* w_codes,
                const uint16_t* w_scales, const float* bias, void* Y, int y_dtype, int64_t ldy,
                int64_t M, int64_t K, int64_t N, int32_t group, void* ws, size_t ws_bytes,
                int32_t activation, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_linear";
  if (int s = check_activation(activation, fn)) return s;
  if (int s = check_common(M, K, R, group, fn)) return s;
  if (!ws) {
    set_error("%s: null workspace", fn);
    return SVDQ_ERR_NULL;
  }
  const WsLayout L = ws_layout(M, K, R, false);
  if (ws_bytes < L.total) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, L.total);
    return SVDQ_ERR_WORKSPACE;
  }
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) {
    set_error("%s: workspace must be 256-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* a_codes = base + L.codes;
  uint16_t* a_scales = reinterpret_cast<uint16_t*>(base + L.scales);
  float* D = R > 0 ? reinterpret_cast<float*>(base + L.d) : nullptr;
  if (int s = validate_k1(X, x_dtype, M, K, ldx, inv_smooth, L1p, R, group, a_codes, a_scales, D,
                          fn))
    return s;
  if (int s = validate_k2(a_codes, a_scales, w_codes, w_scales, D, L2t, R, bias, Y, y_dtype, M, N,
                          K, ldy, group, fn))
    return s;
  if (int s = device_ready()) return s;
  if (int s = check_hip(launch_k1(X, x_dtype == SVDQ_F16, M, K, ldx, inv_smooth, L1p, R, a_codes,
                                  a_scales, false, D, stream),
                        "svdq_linear K1 launch"))
    return s;
  return check_hip(launch_k2(a_codes, a_scales, w_codes, w_scales, D, L2t, R, bias, Y,
                             y_dtype == SVDQ_F16, M, N, K, ldy, activation == SVDQ_ACT_GELU_TANH, stream),
                   "svdq_linear K2 launch");
}

namespace {
// svdq_linear's workspace, then the packed factors L1p (R*K fp16) and L2t
// (N*R fp16)
struct CanonWs {
  WsLayout base;
  size_t l1p, l2t, total;
};
CanonWs canon_ws_layout(int64_t M, int64_t K, int64_t N, int32_t R) {
  CanonWs c;
  c.base = ws_layout(M, K, R, false);
  c.l1p = c.base.total;
  c.l2t = c.l1p + round_up(static_cast<size_t>(R) * K * 2, 256);
  c.total = c.l2t + round_up(static_cast<size_t>(N) * R * 2, 256);
  return c;
}
}  // namespace

size_t svdq_linear_canonical_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t R,
                                             int32_t group) {
  if (M < 1 || N < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0 || group != SVDQ_GROUP || R < 0)
    return 0;
  return canon_ws_layout(M, K, N, R).total;
}

int svdq_linear_canonical(const void* X, int x_dtype, int64_t ldx, const float* inv_smooth,
                          const uint16_t* L1, const uint16_t* L2, int32_t R,
                          const uint8_t* w_codes, const uint16_t* w_scales, const float* bias,
                          void* Y, int y_dtype, int64_t ldy, int64_t M, int64_t K, int64_t N,
                          int32_t group, void* ws, size_t ws_bytes, int32_t activation,
                          hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_linear_canonical";
  if (int s = check_activation(activation, fn)) return s;
  if (int s = check_common(M, K, R, group, fn)) return s;
  if (N < 1) {
    set_error("%s: N=%lld", fn, (long long)N);
    return SVDQ_ERR_SHAPE;
  }
  if (R > 0 && (!L1 || !L2)) {
    set_error("%s: null low-rank factor", fn);
    return SVDQ_ERR_NULL;
  }
  if (R > 0 && (!aligned16(L1) || !aligned16(L2))) {
    set_error("%s: L1 and L2 must be 16-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  if (!ws) {
    set_error("%s: null workspace", fn);
    return SVDQ_ERR_NULL;
  }
  const CanonWs L = canon_ws_layout(M, K, N, R);
  if (ws_bytes < L.total) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, L.total);
    return SVDQ_ERR_WORKSPACE;
  }
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) {
    set_error("%s: workspace must be 256-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* a_codes = base + L.base.codes;
  uint16_t* a_scales = reinterpret_cast<uint16_t*>(base + L.base.scales);
  float* D = R > 0 ? reinterpret_cast<float*>(base + L.base.d) : nullptr;
  uint16_t* L1p = R > 0 ? reinterpret_cast<uint16_t*>(base + L.l1p) : nullptr;
  uint16_t* L2t = R > 0 ? reinterpret_cast<uint16_t*>(base + L.l2t) : nullptr;
  if (int s = validate_k1(X, x_dtype, M, K, ldx, inv_smooth, L1p, R, group, a_codes, a_scales, D,
                          fn))
    return s;
  if (int s = validate_k2(a_codes, a_scales, w_codes, w_scales, D, L2t, R, bias, Y, y_dtype, M, N,
                          K, ldy, group, fn))
    return s;
  if (int s = device_ready()) return s;
  if (R > 0) {
    if (int s = check_hip(launch_pack_lowrank(L1, L2, K, N, R, L1p, L2t, stream),
                          "svdq_linear_canonical factor packing launch"))
      return s;
  }
  if (int s = check_hip(launch_k1(X, x_dtype == SVDQ_F16, M, K, ldx, inv_smooth, L1p, R, a_codes,
                                  a_scales, false, D, stream),
                        "svdq_linear_canonical K1 launch"))
    return s;
  return check_hip(launch_k2(a_codes, a_scales, w_codes, w_scales, D, L2t, R, bias, Y,
                             y_dtype == SVDQ_F16, M, N, K, ldy, activation == SVDQ_ACT_GELU_TANH, stream),
                   "svdq_linear_canonical K2 launch");
}

size_t svdq_quantize_act_workspace_bytes(int64_t M, int64_t K, int32_t R) {
  if (M < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0 || R < 0 || R > SVDQ_MAX_RANK ||
      R % 16 != 0)
    return 0;
  return k1_split_bytes(M, K, R, kK1Int4Tiled, false);
}

namespace {
// The optional workspace of the tiled and MXFP4 pre-kernels: null, or at least
// svdq_quantize_act_workspace_bytes and 256-byte aligned. Returns the partial
// buffer to hand to the launcher (null: run unsplit).
int k1_workspace(void* ws, size_t ws_bytes, int64_t M, int64_t K, int32_t R, int fmt,
                 const char* fn, float** part) {
  *part = nullptr;
  if (ws == nullptr) return SVDQ_OK;
  const size_t need = k1_split_bytes(M, K, R, fmt, false);
  if (ws_bytes < need) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    return SVDQ_ERR_WORKSPACE;
  }
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) {
    set_error("%s: workspace must be 256-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  *part = need > 0 ? static_cast<float*>(ws) : nullptr;
  return SVDQ_OK;
}
}  // namespace

int svdq_quantize_act_lowrank_down_tiled(const void* X, int x_dtype, int64_t M, int64_t K,
                                         int64_t ldx, const float* inv_smooth,
                                         const uint16_t* L1p, int32_t R, uint8_t* a_ops_t,
                                         float* a_scales_t, uint16_t* D_t, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_quantize_act_lowrank_down_tiled";
  // D_t is checked (null, alignment) and passed as an untyped device pointer
  float* D = reinterpret_cast<float*>(D_t);
  if (int s = validate_k1(X, x_dtype, M, K, ldx, inv_smooth, L1p, R, SVDQ_GROUP, a_ops_t,
                          a_scales_t, D, fn))
    return s;
  float* part = nullptr;
  if (int s = k1_workspace(workspace, workspace_bytes, M, K, R, kK1Int4Tiled, fn, &part))
    return s;
  if (int s = device_ready()) return s;
  return check_hip(launch_k1(X, x_dtype == SVDQ_F16, M, K, ldx, inv_smooth, L1p, R, a_ops_t,
                             a_scales_t, kK1Int4Tiled, D, stream, nullptr, part),
                   "svdq_quantize_act_lowrank_down_tiled launch");
}

namespace {
// K2T adds each lane's offset into the tiled weight scales in 32 bits, and
// its grid can hold up to 3 x 1024 more workgroups than tiles (split tails).
int check_k2t_shape(int64_t M, int64_t N, int64_t K, const char* fn) {
  if (((N + 31) / 32) * (K / SVDQ_GROUP) * 256 > int64_t{0xFFFFFFFF} ||
      ((M + 127) / 128) * ((N + 127) / 128) > 0x7FFFFFFF - 4096) {
    set_error("%s: N=%lld K=%lld too large for the tiled kernel", fn, (long long)N, (long long)K);
    return SVDQ_ERR_SHAPE;
  }
  return SVDQ_OK;
}
}  // namespace

size_t svdq_gemm_tiled_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0) return 0;
  return k2t_split_bytes(M, N, K);
}

namespace {
// The optional workspace of the tiled GEMM: null (unsplit), or at least
// svdq_gemm_tiled_workspace_bytes and 256-byte aligned. Returns the partial
// buffer to hand to the launcher (null: run unsplit).
int k2t_workspace(void* ws, size_t ws_bytes, int64_t M, int64_t N, int64_t K, const char* fn,
                  float** part) {
  *part = nullptr;
  if (ws == nullptr) return SVDQ_OK;
  const size_t need = k2t_split_bytes(M, N, K);
  if (ws_bytes < need) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    return SVDQ_ERR_WORKSPACE;
  }
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) {
    set_error("%s: workspace must be 256-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  *part = need > 0 ? static_cast<float*>(ws) : nullptr;
  return SVDQ_OK;
}

// The fused tiled entry points: the tiled GEMM's partials follow the layout's
// `total` bytes when the caller's workspace holds them (else unsplit).
float* k2t_part_after(void* ws, size_t ws_bytes, size_t total, int64_t M, int64_t N, int64_t K) {
  const size_t need = k2t_split_bytes(M, N, K);
  if (need == 0 || ws_bytes < total + need) return nullptr;
  return reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + total);
}
}  // namespace

int svdq_w4a4_gemm_lowrank_up_tiled(const uint8_t* a_ops_t, const float* a_scales_t,
                                    const uint8_t* w_codes_t, const float* w_scales_t,
                                    const uint16_t* D_t, const uint16_t* L2t, int32_t R,
                                    const float* bias, void* Y, int y_dtype, int64_t M, int64_t N,
                                    int64_t K, int64_t ldy, int32_t activation, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_w4a4_gemm_lowrank_up_tiled";
  if (int s = validate_k2(a_ops_t, a_scales_t, w_codes_t, w_scales_t,
                          reinterpret_cast<const float*>(D_t), L2t, R, bias, Y, y_dtype,
                          M, N, K, ldy, SVDQ_GROUP, fn))
    return s;
  if (int s = check_k2t_shape(M, N, K, fn)) return s;
  if (int s = check_activation(activation, fn)) return s;
  float* part = nullptr;
  if (int s = k2t_workspace(workspace, workspace_bytes, M, N, K, fn, &part)) return s;
  if (int s = device_ready()) return s;
  return check_hip(launch_k2t(a_ops_t, a_scales_t, w_codes_t, w_scales_t, D_t, L2t, R, bias, Y,
                              y_dtype == SVDQ_F16, M, N, K, ldy,
                              activation == SVDQ_ACT_GELU_TANH, stream, part),
                   "svdq_w4a4_gemm_lowrank_up_tiled launch");
}

size_t svdq_linear_tiled_workspace_bytes(int64_t M, int64_t K, int32_t R) {
  if (M < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0 || R < 0) return 0;
  return tiled_ws_layout(M, K, R).total;
}

int svdq_linear_tiled(const void* X, int x_dtype, int64_t ldx, const float* inv_smooth,
                      const uint16_t* L1p, const uint16_t* L2t, int32_t R,
                      const uint8_t* w_codes_t, const float* w_scales_t, const float* bias,
                      void* Y, int y_dtype, int64_t ldy, int64_t M, int64_t K, int64_t N,
                      void* ws, size_t ws_bytes, int32_t activation, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_linear_tiled";
  if (int s = check_activation(activation, fn)) return s;
  if (int s = check_common(M, K, R, SVDQ_GROUP, fn)) return s;
  if (!ws) {
    set_error("%s: null workspace", fn);
    return SVDQ_ERR_NULL;
  }
  const WsLayout L = tiled_ws_layout(M, K, R);
  if (ws_bytes < L.total) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, L.total);
    return SVDQ_ERR_WORKSPACE;
  }
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) {
    set_error("%s: workspace must be 256-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* a_ops = base + L.codes;
  float* a_scales = reinterpret_cast<float*>(base + L.scales);
  float* D = R > 0 ? reinterpret_cast<float*>(base + L.d) : nullptr;
  float* part = L.total > L.part ? reinterpret_cast<float*>(base + L.part) : nullptr;
  if (int s = validate_k1(X, x_dtype, M, K, ldx, inv_smooth, L1p, R, SVDQ_GROUP, a_ops, a_scales,
                          D, fn))
    return s;
  if (int s = validate_k2(a_ops, a_scales, w_codes_t, w_scales_t, D, L2t, R, bias, Y, y_dtype, M,
                          N, K, ldy, SVDQ_GROUP, fn))
    return s;
  if (int s = check_k2t_shape(M, N, K, fn)) return s;
  if (int s = device_ready()) return s;
  if (int s = check_hip(launch_k1(X, x_dtype == SVDQ_F16, M, K, ldx, inv_smooth, L1p, R, a_ops,
                                  a_scales, kK1Int4Tiled, D, stream, nullptr, part),
                        "svdq_linear_tiled K1 launch"))
    return s;
  return check_hip(launch_k2t(a_ops, a_scales, w_codes_t, w_scales_t,
                              reinterpret_cast<const uint16_t*>(D), L2t, R, bias, Y,
                              y_dtype == SVDQ_F16, M, N, K, ldy, activation == SVDQ_ACT_GELU_TANH,
                              stream, k2t_part_after(ws, ws_bytes, L.total, M, N, K)),
                   "svdq_linear_tiled K2 launch");
}

int svdq_quantize_act_lowrank_down_mx(const void* X, int x_dtype, int64_t M, int64_t K,
                                      int64_t ldx, const float* inv_smooth, const uint16_t* L1p,
                                      int32_t R, uint8_t* a_codes, uint8_t* a_e8m0,
                                      uint16_t* D_t, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_quantize_act_lowrank_down_mx";
  float* D = reinterpret_cast<float*>(D_t);   // checked for null and alignment only
  if (int s = validate_k1(X, x_dtype, M, K, ldx, inv_smooth, L1p, R, SVDQ_GROUP, a_codes, a_e8m0,
                          D, fn))
    return s;
  float* part = nullptr;
  if (int s = k1_workspace(workspace, workspace_bytes, M, K, R, kK1Mx, fn, &part)) return s;
  if (int s = device_ready()) return s;
  return check_hip(launch_k1(X, x_dtype == SVDQ_F16, M, K, ldx, inv_smooth, L1p, R, a_codes,
                             a_e8m0, kK1Mx, D, stream, nullptr, part),
                   "svdq_quantize_act_lowrank_down_mx launch");
}

int svdq_mx_gemm_lowrank_up(const uint8_t* a_codes, const uint8_t* a_e8m0,
                            const uint8_t* w_codes, const uint8_t* w_e8m0, const uint16_t* D_t,
                            const uint16_t* L2t, int32_t R, const float* bias, void* Y,
                            int y_dtype, int64_t M, int64_t N, int64_t K, int64_t ldy,
                            int32_t activation, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_mx_gemm_lowrank_up";
  if (int s = validate_k2(a_codes, a_e8m0, w_codes, w_e8m0, reinterpret_cast<const float*>(D_t),
                          L2t, R, bias, Y, y_dtype, M, N, K, ldy, SVDQ_GROUP, fn))
    return s;
  if (int s = check_activation(activation, fn)) return s;
  if (int s = device_ready()) return s;
  return check_hip(launch_k2_mx(a_codes, a_e8m0, w_codes, w_e8m0, D_t, L2t, R, bias, Y,
                                y_dtype == SVDQ_F16, M, N, K, ldy,
                                activation == SVDQ_ACT_GELU_TANH, stream),
                   "svdq_mx_gemm_lowrank_up launch");
}

size_t svdq_linear_mx_workspace_bytes(int64_t M, int64_t K, int32_t R) {
  if (M < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0 || R < 0) return 0;
  return ws_layout(M, K, R, true).total;
}

int svdq_linear_mx(const void* X, int x_dtype, int64_t ldx, const float* inv_smooth,
                   const uint16_t* L1p, const uint16_t* L2t, int32_t R, const uint8_t* w_codes,
                   const uint8_t* w_e8m0, const float* bias, void* Y, int y_dtype, int64_t ldy,
                   int64_t M, int64_t K, int64_t N, void* ws, size_t ws_bytes,
                   int32_t activation, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_linear_mx";
  if (int s = check_activation(activation, fn)) return s;
  if (!ws) {
    set_error("%s: null workspace", fn);
    return SVDQ_ERR_NULL;
  }
  if (int s = check_common(M, K, R, SVDQ_GROUP, fn)) return s;
  const WsLayout L = ws_layout(M, K, R, true);
  if (ws_bytes < L.total) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, L.total);
    return SVDQ_ERR_WORKSPACE;
  }
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) {
    set_error("%s: workspace must be 256-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* a_codes = base + L.codes;
  uint8_t* a_e8m0 = base + L.scales;
  float* D = R > 0 ? reinterpret_cast<float*>(base + L.d) : nullptr;
  float* part = L.total > L.part ? reinterpret_cast<float*>(base + L.part) : nullptr;
  if (int s = validate_k1(X, x_dtype, M, K, ldx, inv_smooth, L1p, R, SVDQ_GROUP, a_codes, a_e8m0,
                          D, fn))
    return s;
  if (int s = validate_k2(a_codes, a_e8m0, w_codes, w_e8m0, D, L2t, R, bias, Y, y_dtype, M, N, K,
                          ldy, SVDQ_GROUP, fn))
    return s;
  if (int s = device_ready()) return s;
  if (int s = check_hip(launch_k1(X, x_dtype == SVDQ_F16, M, K, ldx, inv_smooth, L1p, R, a_codes,
                                  a_e8m0, kK1Mx, D, stream, nullptr, part),
                        "svdq_linear_mx K1 launch"))
    return s;
  return check_hip(launch_k2_mx(a_codes, a_e8m0, w_codes, w_e8m0,
                                reinterpret_cast<const uint16_t*>(D), L2t, R, bias, Y,
                                y_dtype == SVDQ_F16, M, N, K, ldy,
                                activation == SVDQ_ACT_GELU_TANH, stream),
                   "svdq_linear_mx K2 launch");
}

int svdq_quantize_act_lowrank_down_conv(const void* X, int x_dtype, int64_t batch, int64_t H,
                                        int64_t W, int64_t C, int32_t KH, int32_t KW,
                                        int32_t stride, int32_t pad, const float* inv_smooth,
                                        const uint16_t* L1p, int32_t R, uint8_t* a_codes,
                                        uint16_t* a_scales, float* D, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_quantize_act_lowrank_down_conv";
  ConvShape cs;
  if (int s = check_conv(batch, H, W, C, KH, KW, stride, pad, cs, fn)) return s;
  if (int s = validate_k1(X, x_dtype, cs.M, cs.K, cs.K, inv_smooth, L1p, R, SVDQ_GROUP, a_codes,
                          a_scales, D, fn))
    return s;
  if (int s = device_ready()) return s;
  const ConvGeom g = conv_geom(cs);
  return check_hip(launch_k1(X, x_dtype == SVDQ_F16, cs.M, cs.K, cs.K, inv_smooth, L1p, R,
                             a_codes, a_scales, false, D, stream, &g),
                   "svdq_quantize_act_lowrank_down_conv launch");
}

int svdq_conv2d(const void* X, int x_dtype, int64_t batch, int64_t H, int64_t W, int64_t C,
                int32_t KH, int32_t KW, int32_t stride, int32_t pad, const float* inv_smooth,
                const uint16_t* L1p, const uint16_t* L2t, int32_t R, const uint8_t* w_codes,
                const uint16_t* w_scales, const float* bias, void* Y, int y_dtype, int64_t N,
                void* ws, size_t ws_bytes, int32_t activation, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_conv2d";
  if (int s = check_activation(activation, fn)) return s;
  if (!ws) {
    set_error("%s: null workspace", fn);
    return SVDQ_ERR_NULL;
  }
  ConvShape cs;
  if (int s = check_conv(batch, H, W, C, KH, KW, stride, pad, cs, fn)) return s;
  if (int s = check_common(cs.M, cs.K, R, SVDQ_GROUP, fn)) return s;
  const WsLayout L = ws_layout(cs.M, cs.K, R, false);
  if (ws_bytes < L.total) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, L.total);
    return SVDQ_ERR_WORKSPACE;
  }
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) {
    set_error("%s: workspace must be 256-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* a_codes = base + L.codes;
  uint16_t* a_scales = reinterpret_cast<uint16_t*>(base + L.scales);
  float* D = R > 0 ? reinterpret_cast<float*>(base + L.d) : nullptr;
  if (int s = validate_k1(X, x_dtype, cs.M, cs.K, cs.K, inv_smooth, L1p, R, SVDQ_GROUP, a_codes,
                          a_scales, D, fn))
    return s;
  if (int s = validate_k2(a_codes, a_scales, w_codes, w_scales, D, L2t, R, bias, Y, y_dtype, cs.M,
                          N, cs.K, N, SVDQ_GROUP, fn))
    return s;
  if (int s = device_ready()) return s;
  const ConvGeom g = conv_geom(cs);
  if (int s = check_hip(launch_k1(X, x_dtype == SVDQ_F16, cs.M, cs.K, cs.K, inv_smooth, L1p, R,
                                  a_codes, a_scales, false, D, stream, &g),
                        "svdq_conv2d K1 launch"))
    return s;
  return check_hip(launch_k2(a_codes, a_scales, w_codes, w_scales, D, L2t, R, bias, Y,
                             y_dtype == SVDQ_F16, cs.M, N, cs.K, N,
                             activation == SVDQ_ACT_GELU_TANH, stream),
                   "svdq_conv2d K2 launch");
}

int svdq_quantize_act_lowrank_down_conv_tiled(const void* X, int x_dtype, int64_t batch,
                                              int64_t H, int64_t W, int64_t C, int32_t KH,
                                              int32_t KW, int32_t stride, int32_t pad,
                                              const float* inv_smooth, const uint16_t* L1p,
                                              int32_t R, uint8_t* a_ops_t, float* a_scales_t,
                                              uint16_t* D_t, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_quantize_act_lowrank_down_conv_tiled";
  float* D = reinterpret_cast<float*>(D_t);   // checked for null and alignment only
  ConvShape cs;
  if (int s = check_conv(batch, H, W, C, KH, KW, stride, pad, cs, fn)) return s;
  if (int s = validate_k1(X, x_dtype, cs.M, cs.K, cs.K, inv_smooth, L1p, R, SVDQ_GROUP, a_ops_t,
                          a_scales_t, D, fn))
    return s;
  if (int s = device_ready()) return s;
  const ConvGeom g = conv_geom(cs);
  return check_hip(launch_k1(X, x_dtype == SVDQ_F16, cs.M, cs.K, cs.K, inv_smooth, L1p, R,
                             a_ops_t, a_scales_t, kK1Int4Tiled, D, stream, &g),
                   "svdq_quantize_act_lowrank_down_conv_tiled launch");
}

int svdq_conv2d_tiled(const void* X, int x_dtype, int64_t batch, int64_t H, int64_t W, int64_t C,
                      int32_t KH, int32_t KW, int32_t stride, int32_t pad,
                      const float* inv_smooth, const uint16_t* L1p, const uint16_t* L2t,
                      int32_t R, const uint8_t* w_codes_t, const float* w_scales_t,
                      const float* bias, void* Y, int y_dtype, int64_t N, void* ws,
                      size_t ws_bytes, int32_t activation, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_conv2d_tiled";
  if (int s = check_activation(activation, fn)) return s;
  if (!ws) {
    set_error("%s: null workspace", fn);
    return SVDQ_ERR_NULL;
  }
  ConvShape cs;
  if (int s = check_conv(batch, H, W, C, KH, KW, stride, pad, cs, fn)) return s;
  if (int s = check_common(cs.M, cs.K, R, SVDQ_GROUP, fn)) return s;
  const WsLayout L = tiled_ws_layout(cs.M, cs.K, R);
  if (ws_bytes < L.total) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, L.total);
    return SVDQ_ERR_WORKSPACE;
  }
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) {
    set_error("%s: workspace must be 256-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* a_ops = base + L.codes;
  float* a_scales = reinterpret_cast<float*>(base + L.scales);
  float* D = R > 0 ? reinterpret_cast<float*>(base + L.d) : nullptr;
  if (int s = validate_k1(X, x_dtype, cs.M, cs.K, cs.K, inv_smooth, L1p, R, SVDQ_GROUP, a_ops,
                          a_scales, D, fn))
    return s;
  if (int s = validate_k2(a_ops, a_scales, w_codes_t, w_scales_t, D, L2t, R, bias, Y, y_dtype,
                          cs.M, N, cs.K, N, SVDQ_GROUP, fn))
    return s;
  if (int s = check_k2t_shape(cs.M, N, cs.K, fn)) return s;
  if (int s = device_ready()) return s;
  const ConvGeom g = conv_geom(cs);
  if (int s = check_hip(launch_k1(X, x_dtype == SVDQ_F16, cs.M, cs.K, cs.K, inv_smooth, L1p, R,
                                  a_ops, a_scales, kK1Int4Tiled, D, stream, &g),
                        "svdq_conv2d_tiled K1 launch"))
    return s;
  return check_hip(launch_k2t(a_ops, a_scales, w_codes_t, w_scales_t,
                              reinterpret_cast<const uint16_t*>(D), L2t, R, bias, Y,
                              y_dtype == SVDQ_F16, cs.M, N, cs.K, N,
                              activation == SVDQ_ACT_GELU_TANH, stream,
                              k2t_part_after(ws, ws_bytes, L.total, cs.M, N, cs.K)),
                   "svdq_conv2d_tiled K2 launch");
}

int svdq_quantize_act_lowrank_down_conv_mx(const void* X, int x_dtype, int64_t batch, int64_t H,
                                           int64_t W, int64_t C, int32_t KH, int32_t KW,
                                           int32_t stride, int32_t pad, const float* inv_smooth,
                                           const uint16_t* L1p, int32_t R, uint8_t* a_codes_t,
                                           uint8_t* a_exps_t, uint16_t* D_t, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_quantize_act_lowrank_down_conv_mx";
  float* D = reinterpret_cast<float*>(D_t);   // checked for null and alignment only
  ConvShape cs;
  if (int s = check_conv(batch, H, W, C, KH, KW, stride, pad, cs, fn)) return s;
  if (int s = validate_k1(X, x_dtype, cs.M, cs.K, cs.K, inv_smooth, L1p, R, SVDQ_GROUP, a_codes_t,
                          a_exps_t, D, fn))
    return s;
  if (int s = device_ready()) return s;
  const ConvGeom g = conv_geom(cs);
  return check_hip(launch_k1(X, x_dtype == SVDQ_F16, cs.M, cs.K, cs.K, inv_smooth, L1p, R,
                             a_codes_t, a_exps_t, true, D, stream, &g),
                   "svdq_quantize_act_lowrank_down_conv_mx launch");
}

int svdq_conv2d_mx(const void* X, int x_dtype, int64_t batch, int64_t H, int64_t W, int64_t C,
                   int32_t KH, int32_t KW, int32_t stride, int32_t pad, const float* inv_smooth,
                   const uint16_t* L1p, const uint16_t* L2t, int32_t R, const uint8_t* w_codes_t,
                   const uint8_t* w_exps_t, const float* bias, void* Y, int y_dtype, int64_t N,
                   void* ws, size_t ws_bytes, int32_t activation, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_conv2d_mx";
  if (int s = check_activation(activation, fn)) return s;
  if (!ws) {
    set_error("%s: null workspace", fn);
    return SVDQ_ERR_NULL;
  }
  ConvShape cs;
  if (int s = check_conv(batch, H, W, C, KH, KW, stride, pad, cs, fn)) return s;
  if (int s = check_common(cs.M, cs.K, R, SVDQ_GROUP, fn)) return s;
  const WsLayout L = ws_layout(cs.M, cs.K, R, true);
  if (ws_bytes < L.total) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, L.total);
    return SVDQ_ERR_WORKSPACE;
  }
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) {
    set_error("%s: workspace must be 256-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  uint8_t* base = static_cast<uint8_t*>(ws);
  uint8_t* a_codes = base + L.codes;
  uint8_t* a_exps = base + L.scales;
  float* D = R > 0 ? reinterpret_cast<float*>(base + L.d) : nullptr;
  if (int s = validate_k1(X, x_dtype, cs.M, cs.K, cs.K, inv_smooth, L1p, R, SVDQ_GROUP, a_codes,
                          a_exps, D, fn))
    return s;
  if (int s = validate_k2(a_codes, a_exps, w_codes_t, w_exps_t, D, L2t, R, bias, Y, y_dtype, cs.M,
                          N, cs.K, N, SVDQ_GROUP, fn))
    return s;
  if (int s = device_ready()) return s;
  const ConvGeom g = conv_geom(cs);
  if (int s = check_hip(launch_k1(X, x_dtype == SVDQ_F16, cs.M, cs.K, cs.K, inv_smooth, L1p, R,
                                  a_codes, a_exps, true, D, stream, &g),
                        "svdq_conv2d_mx K1 launch"))
    return s;
  return check_hip(launch_k2_mx(a_codes, a_exps, w_codes_t, w_exps_t,
                                reinterpret_cast<const uint16_t*>(D), L2t, R, bias, Y,
                                y_dtype == SVDQ_F16, cs.M, N, cs.K, N,
                                activation == SVDQ_ACT_GELU_TANH, stream),
                   "svdq_conv2d_mx K2 launch");
}

size_t svdq_w4a16_x_tiled_bytes(int64_t M, int64_t K) {
  if (M < 1 || K < SVDQ_GROUP || K % SVDQ_GROUP != 0) return 0;
  return static_cast<size_t>((M + 15) / 16) * static_cast<size_t>(K / 32) * 1024;
}

namespace {

int validate_w4a16_x(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                     const void* x_t, const char* fn) {
  if (!X || !x_t) {
    set_error("%s: null pointer", fn);
    return SVDQ_ERR_NULL;
  }
  if (!known_dtype(x_dtype)) {
    set_error("%s: x_dtype %d", fn, x_dtype);
    return SVDQ_ERR_DTYPE;
  }
  if (int s = check_common(M, K, 0, SVDQ_GROUP, fn)) return s;
  if (ldx < K || (M + 15) / 16 > 0x7FFFFFFF) {
    set_error("%s: ldx=%lld < K=%lld", fn, (long long)ldx, (long long)K);
    return SVDQ_ERR_SHAPE;
  }
  if (!aligned16(X) || !aligned16(x_t) || (ldx * esize(x_dtype)) % 16 != 0) {
    set_error("%s: X, its row stride and x_t must be 16-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  return SVDQ_OK;
}

int validate_w4a16_gemm(const uint16_t* x_t, const uint8_t* wc, const uint16_t* ws,
                        const float* bias, const void* Y, int y_dtype, int64_t M, int64_t N,
                        int64_t K, int64_t ldy, const char* fn) {
  if (!x_t || !wc || !ws || !Y) {
    set_error("%s: null pointer", fn);
    return SVDQ_ERR_NULL;
  }
  if (!known_dtype(y_dtype)) {
    set_error("%s: y_dtype %d", fn, y_dtype);
    return SVDQ_ERR_DTYPE;
  }
  if (int s = check_common(M, K, 0, SVDQ_GROUP, fn)) return s;
  if (N < 1 || ldy < N || ((M + 127) / 128) * ((N + 255) / 256) > 0x7FFFFFFF) {
    set_error("%s: N=%lld ldy=%lld", fn, (long long)N, (long long)ldy);
    return SVDQ_ERR_SHAPE;
  }
  if (!aligned16(x_t) || !aligned16(wc) || !aligned16(ws)) {
    set_error("%s: x_t and the tiled weights must be 16-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  if ((reinterpret_cast<uintptr_t>(Y) % esize(y_dtype)) != 0 ||
      (bias && (reinterpret_cast<uintptr_t>(bias) & 3u) != 0)) {
    set_error("%s: Y and bias must be aligned to their element size", fn);
    return SVDQ_ERR_ALIGN;
  }
  return SVDQ_OK;
}

}  // namespace

int svdq_w4a16_tile_activation(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                               uint16_t* x_t, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_w4a16_tile_activation";
  if (int s = validate_w4a16_x(X, x_dtype, M, K, ldx, x_t, fn)) return s;
  if (int s = device_ready()) return s;
  return check_hip(launch_w4a16_tile_x(X, x_dtype == SVDQ_F16, M, K, ldx, x_t, stream),
                   "svdq_w4a16_tile_activation launch");
}

int svdq_w4a16_gemm(const uint16_t* x_t, const uint8_t* w_codes_t, const uint16_t* w_scales_t,
                    const float* bias, void* Y, int y_dtype, int64_t M, int64_t N, int64_t K,
                    int64_t ldy, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_w4a16_gemm";
  if (int s = validate_w4a16_gemm(x_t, w_codes_t, w_scales_t, bias, Y, y_dtype, M, N, K, ldy, fn))
    return s;
  if (int s = device_ready()) return s;
  return check_hip(launch_w4a16_gemm(x_t, w_codes_t, w_scales_t, bias, Y, y_dtype == SVDQ_F16, M,
                                     N, K, ldy, stream),
                   "svdq_w4a16_gemm launch");
}

int svdq_linear_w4a16(const void* X, int x_dtype, int64_t ldx, const uint8_t* w_codes_t,
                      const uint16_t* w_scales_t, const float* bias, void* Y, int y_dtype,
                      int64_t ldy, int64_t M, int64_t K, int64_t N, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_linear_w4a16";
  if (!ws) {
    set_error("%s: null workspace", fn);
    return SVDQ_ERR_NULL;
  }
  if (int s = check_common(M, K, 0, SVDQ_GROUP, fn)) return s;
  const size_t need = svdq_w4a16_x_tiled_bytes(M, K);
  if (ws_bytes < need) {
    set_error("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
    return SVDQ_ERR_WORKSPACE;
  }
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) {
    set_error("%s: workspace must be 256-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  uint16_t* x_t = static_cast<uint16_t*>(ws);
  if (int s = validate_w4a16_x(X, x_dtype, M, K, ldx, x_t, fn)) return s;
  if (int s = validate_w4a16_gemm(x_t, w_codes_t, w_scales_t, bias, Y, y_dtype, M, N, K, ldy, fn))
    return s;
  if (int s = device_ready()) return s;
  if (int s = check_hip(launch_w4a16_tile_x(X, x_dtype == SVDQ_F16, M, K, ldx, x_t, stream),
                        "svdq_linear_w4a16 tiling launch"))
    return s;
  return check_hip(launch_w4a16_gemm(x_t, w_codes_t, w_scales_t, bias, Y, y_dtype == SVDQ_F16, M,
                                     N, K, ldy, stream),
                   "svdq_linear_w4a16 GEMM launch");
}

int svdq_debug_group_partials(const uint8_t* a_codes, const uint8_t* w_codes, int64_t M, int64_t N,
                              int64_t K, int32_t group, int64_t row0, int64_t rows, int32_t* P,
                              hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_debug_group_partials";
  if (!a_codes || !w_codes || !P) {
    set_error("%s: null pointer", fn);
    return SVDQ_ERR_NULL;
  }
  if (int s = check_common(M, K, 0, group, fn)) return s;
  if (N < 1 || row0 < 0 || rows < 1 || row0 + rows > M || (rows + 15) / 16 > 0x7FFFFFFF ||
      (N + 15) / 16 > 65535) {
    set_error("%s: N=%lld row0=%lld rows=%lld M=%lld", fn, (long long)N, (long long)row0,
              (long long)rows, (long long)M);
    return SVDQ_ERR_SHAPE;
  }
  if (!aligned16(a_codes) || !aligned16(w_codes) || !aligned16(P)) {
    set_error("%s: device pointers must be 16-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  if (int s = device_ready()) return s;
  return check_hip(launch_debug_partials(a_codes, w_codes, M, N, K, row0, rows, P, stream),
                   "svdq_debug_group_partials launch");
}

int svdq_clock_rates(int32_t* wall_khz, int32_t* peak_khz) {
  clear_error();
  if (!wall_khz || !peak_khz) {
    set_error("svdq_clock_rates: null pointer");
    return SVDQ_ERR_NULL;
  }
  if (int s = device_ready()) return s;
  int dev = 0;
  if (int s = check_hip(hipGetDevice(&dev), "svdq_clock_rates")) return s;
  int w = 0, c = 0;
  if (int s = check_hip(hipDeviceGetAttribute(&w, hipDeviceAttributeWallClockRate, dev),
                        "svdq_clock_rates wall clock"))
    return s;
  if (int s = check_hip(hipDeviceGetAttribute(&c, hipDeviceAttributeClockRate, dev),
                        "svdq_clock_rates shader clock"))
    return s;
  *wall_khz = w;
  *peak_khz = c;
  return SVDQ_OK;
}

int svdq_clock_probe(uint64_t* samples, int32_t max_samples, int64_t interval_ticks,
                     const int32_t* stop, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_clock_probe";
  if (!samples || !stop) {
    set_error("%s: null pointer", fn);
    return SVDQ_ERR_NULL;
  }
  if ((reinterpret_cast<uintptr_t>(samples) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(stop) & 3u) != 0) {
    set_error("%s: samples must be 8-byte and stop 4-byte aligned", fn);
    return SVDQ_ERR_ALIGN;
  }
  int32_t wall = 0, peak = 0;
  if (int s = svdq_clock_rates(&wall, &peak)) return s;
  // at most 10 ms between samples and 60 s in all, in ticks of the wall counter
  const int64_t per_ms = wall > 0 ? wall : 100000;
  if (max_samples < 1 || max_samples > (1 << 20) || interval_ticks < 1 ||
      interval_ticks > 10 * per_ms || interval_ticks * max_samples > 60000 * per_ms) {
    set_error("%s: max_samples=%d interval=%lld out of range", fn, max_samples,
              (long long)interval_ticks);
    return SVDQ_ERR_SHAPE;
  }
  return check_hip(launch_clock_probe(samples, max_samples, interval_ticks, stop, stream),
                   "svdq_clock_probe launch");
}

int svdq_clock_mark(uint64_t* stamp, int32_t* stop, hipStream_t stream) {
  clear_error();
  if (!stamp) {
    set_error("svdq_clock_mark: null pointer");
    return SVDQ_ERR_NULL;
  }
  if ((reinterpret_cast<uintptr_t>(stamp) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(stop) & 3u) != 0) {
    set_error("svdq_clock_mark: stamp must be 8-byte and stop 4-byte aligned");
    return SVDQ_ERR_ALIGN;
  }
  if (int s = device_ready()) return s;
  return check_hip(launch_clock_mark(stamp, stop, stream), "svdq_clock_mark launch");
}

int svdq_gelu_tanh_f16(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t stream) {
  clear_error();
  if (!x || !y) {
    set_error("svdq_gelu_tanh_f16: null pointer");
    return SVDQ_ERR_NULL;
  }
  if (n < 0) {
    set_error("svdq_gelu_tanh_f16: n=%lld", (long long)n);
    return SVDQ_ERR_SHAPE;
  }
  if (!aligned16(x) || !aligned16(y)) {
    set_error("svdq_gelu_tanh_f16: pointers must be 16-byte aligned");
    return SVDQ_ERR_ALIGN;
  }
  if (n == 0) return SVDQ_OK;
  if (int s = device_ready()) return s;
  return check_hip(launch_gelu_f16(x, y, n, stream), "svdq_gelu_tanh_f16 launch");
}

}  // extern "C"
