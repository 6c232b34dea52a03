// Measurement utility (not part of the method): the shader clock the kernels
// run at, sampled while they run.
//
// clock_probe_kernel: one wave, launched on a side stream before a timed
// region, reads the shader-clock cycle counter (clock64) and the constant-rate
// wall counter (wall_clock64) every `interval` wall ticks and stores the pairs.
// It stops when `stop` becomes nonzero or after `max_samples` samples,
// whichever comes first, so it always ends. The ratio of cycle-counter to
// wall-counter increments, times the wall counter's rate, is the shader clock.
//
// clock_mark_kernel: one wave on the timed stream stores the wall counter (the
// edge of the timed region) and, optionally, sets `stop`.
//
// The flag and the samples live in device memory; the flag is read and written
// with agent-scope atomics so the probe, which may run on another XCD, sees it.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace svdq {

namespace {

__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* __restrict__ samples,
                                                         int32_t max_samples, int64_t interval,
                                                         const int32_t* __restrict__ stop) {
  const int lane = threadIdx.x;
  int32_t n = 0;
  for (; n < max_samples; ++n) {
    const uint64_t w0 = static_cast<uint64_t>(wall_clock64());
    const uint64_t c0 = static_cast<uint64_t>(clock64());
    if (lane < 2) samples[2 * n + 1 + lane] = lane == 0 ? c0 : w0;
    if (__hip_atomic_load(stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) {
      ++n;
      break;
    }
    while (static_cast<int64_t>(static_cast<uint64_t>(wall_clock64()) - w0) < interval)
      __builtin_amdgcn_s_sleep(4);
  }
  if (lane == 0) samples[0] = static_cast<uint64_t>(n);
}

__global__ __launch_bounds__(64) void clock_mark_kernel(uint64_t* __restrict__ stamp,
                                                        int32_t* __restrict__ stop) {
  const int lane = threadIdx.x;
  const uint64_t w = static_cast<uint64_t>(wall_clock64());
  if (lane == 0) *stamp = w;
  if (lane == 0 && stop != nullptr)
    __hip_atomic_store(stop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_clock_probe(uint64_t* samples, int32_t max_samples, int64_t interval,
                              const int32_t* stop, hipStream_t stream) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, samples, max_samples,
                     interval, stop);
  return hipGetLastError();
}

hipError_t launch_clock_mark(uint64_t* stamp, int32_t* stop, hipStream_t stream) {
  hipLaunchKernelGGL(clock_mark_kernel, dim3(1), dim3(64), 0, stream, stamp, stop);
  return hipGetLastError();
}

}  // namespace svdq
