// Top-k routing over router logits: one wavefront per token (route_dev.h).
#include "common.h"
#include "kernels.h"
#include "route_dev.h"

namespace bitmoe {

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ gates) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<VPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, gates + (size_t)t * k, nullptr);
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  const int vpl = (E + kWave - 1) / kWave;
  if (vpl <= 1) route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (vpl <= 2) route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (vpl <= 4) route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (vpl <= 6) route_kernel<6><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (vpl <= 8) route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else route_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace bitmoe
