// GELU (tanh form) between the up- and down-projection of a DiT MLP, in
// place or out of place on fp16 data. The pages do not describe this op; it
// is the textbook formula 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))),
// evaluated in fp32 and rounded once to fp16. HBM-bound: 16-byte loads and
// stores, 8 values per thread.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "device_launch.hpp"

namespace svdq {

namespace {

__global__ __launch_bounds__(256) void gelu_f16_kernel(const uint16_t* __restrict__ x,
                                                       uint16_t* __restrict__ y, int64_t n) {
  const int64_t nvec = n / 8;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < nvec;
       i += stride) {
    uint4 v = reinterpret_cast<const uint4*>(x)[i];
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = gelu_tanh_f32(h2f(static_cast<uint16_t>(w[k] & 0xFFFFu)));
      const float b = gelu_tanh_f32(h2f(static_cast<uint16_t>(w[k] >> 16)));
      w[k] = static_cast<uint32_t>(f2h(a)) | (static_cast<uint32_t>(f2h(b)) << 16);
    }
    reinterpret_cast<uint4*>(y)[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  // tail (n % 8 values), handled by the first threads of block 0
  if (blockIdx.x == 0) {
    const int64_t t = nvec * 8 + threadIdx.x;
    if (t < n) y[t] = f2h(gelu_tanh_f32(h2f(x[t])));
  }
}

}  // namespace

hipError_t launch_gelu_f16(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t stream) {
  const int64_t nvec = n / 8;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(gelu_f16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     x, y, n);
  return hipGetLastError();
}

}  // namespace svdq
