// svdq_linear_noalloc: the whole layer (K1 then K2) for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid it). svdq_linear keeps its intermediates (the
// activation codes, scales and D) in a caller workspace; this entry point keeps
// them in `scratch`, a static device array of SVDQ_NOALLOC_MAX_BYTES that the
// code object carries: each GPU the library runs on holds its own copy until
// the process ends, and every call on that GPU shares it. K1 writes every byte
// of it that K2 then reads, so nothing in it has to start at zero; but calls
// that overlap on one GPU (other streams, other threads) race on it and must
// be serialized by the caller.
//
// On the host the name `scratch` is only a stand-in registered with the
// runtime, not a device address: passing it to a kernel would fault. Its
// device address is fetched with hipGetSymbolAddress once per device, with
// that device current, and only that address is ever used.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <mutex>

#include "../../include/svdq.h"
#include "host_internal.hpp"

using namespace svdq;

namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(SVDQ_NOALLOC_MAX_BYTES);
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// Device address of this device's copy of `scratch` (fetched on first use).
int scratch_for_current_device(void** out, const char* fn) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    set_error("%s: no usable GPU: %s", fn, hipGetErrorString(e));
    return SVDQ_ERR_NO_DEVICE;
  }
  if (dev >= kMaxDevices) {
    set_error("%s: device %d beyond the %d the library tracks", fn, dev, kMaxDevices);
    return SVDQ_ERR_NO_DEVICE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t s = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s != hipSuccess) {
      set_error("%s: hipGetSymbolAddress: %s", fn, hipGetErrorString(s));
      return SVDQ_ERR_HIP;
    }
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) {
      set_error("%s: static buffer at %p (need a 256-byte aligned device address)", fn, p);
      return SVDQ_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SVDQ_OK;
}

// Re-label svdq_linear's message with this entry point's name.
void relabel_error(const char* fn) {
  char msg[400];
  std::snprintf(msg, sizeof(msg), "%s", svdq_last_error());
  set_error("%s: %s", fn, msg);
}

}  // namespace

extern "C" int svdq_linear_noalloc(const void* X, int x_dtype, int64_t ldx,
                                   const float* inv_smooth, const uint16_t* L1p,
                                   const uint16_t* L2t, int32_t R, const uint8_t* w_codes,
                                   const uint16_t* w_scales, const float* bias, void* Y,
                                   int y_dtype, int64_t ldy, int64_t M, int64_t K, int64_t N,
                                   int32_t group, int32_t activation, hipStream_t stream) {
  clear_error();
  const char* fn = "svdq_linear_noalloc";
  const size_t need = svdq_linear_workspace_bytes(M, K, R, group);
  if (need == 0) {
    // sizes svdq_linear rejects before it looks at the workspace: let it say which
    const int s = svdq_linear(X, x_dtype, ldx, inv_smooth, L1p, L2t, R, w_codes, w_scales, bias,
                              Y, y_dtype, ldy, M, K, N, group, nullptr, 0, activation, stream);
    relabel_error(fn);
    return s != SVDQ_OK ? s : SVDQ_ERR_SHAPE;
  }
  if (need > kScratchBytes) {
    set_error("%s: the layer needs %zu bytes of intermediates, more than the %zu of the static "
              "buffer", fn, need, kScratchBytes);
    return SVDQ_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if (int s = scratch_for_current_device(&ws, fn)) return s;
  const int s = svdq_linear(X, x_dtype, ldx, inv_smooth, L1p, L2t, R, w_codes, w_scales, bias, Y,
                            y_dtype, ldy, M, K, N, group, ws, kScratchBytes, activation, stream);
  if (s != SVDQ_OK) relabel_error(fn);
  return s;
}
