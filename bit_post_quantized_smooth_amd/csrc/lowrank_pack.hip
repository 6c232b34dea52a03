// The low-rank factors as the method states them, L1 (K x R) and L2 (R x N),
// fp16 row-major (the 16-bit low-rank branch of the SVD split: chattools.cn
// overview, section "SVDQuant的技术原理"), rearranged on the device into the
// operand orders the two kernels read: L1p (K1's down-projection operands)
// and L2t (N x R, K2's up-projection operands). A layout only, no arithmetic:
// every output element is one input element. Small (R (K + N) values), so a
// plain element-per-thread gather.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "device_launch.hpp"

namespace svdq {

namespace {

// L1p element i = (((g * R/16 + c) * 2 + h) * 64 + 16 q + rl) * 8 + j holds
// L1[64 g + 16 q + 8 h + j][16 c + rl]; L2t element n * R + r holds L2[r][n].
__global__ __launch_bounds__(256) void pack_lowrank_kernel(const uint16_t* __restrict__ L1,
                                                           const uint16_t* __restrict__ L2,
                                                           int64_t K, int64_t N, int R,
                                                           uint16_t* __restrict__ L1p,
                                                           uint16_t* __restrict__ L2t) {
  const int64_t n1 = K * R, total = n1 + N * R;
  const int64_t ncb = R / 16;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += stride) {
    if (i < n1) {
      const int64_t j = i & 7, lane = (i >> 3) & 63, h = (i >> 9) & 1, gc = i >> 10;
      const int64_t c = gc % ncb, g = gc / ncb;
      const int64_t k = 64 * g + 16 * (lane >> 4) + 8 * h + j, r = 16 * c + (lane & 15);
      L1p[i] = L1[k * R + r];
    } else {
      const int64_t t = i - n1, n = t / R, r = t % R;
      L2t[t] = L2[r * N + n];
    }
  }
}

}  // namespace

hipError_t launch_pack_lowrank(const uint16_t* L1, const uint16_t* L2, int64_t K, int64_t N,
                               int R, uint16_t* L1p, uint16_t* L2t, hipStream_t stream) {
  const int64_t total = (K + N) * R;
  const int64_t blocks = (total + 255) / 256;
  const dim3 grid(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), block(256);
  hipLaunchKernelGGL(pack_lowrank_kernel, grid, block, 0, stream, L1, L2, K, N, R, L1p, L2t);
  return hipGetLastError();
}

}  // namespace svdq
