// Top-k routing over router logits: one wavefront per token.
//
// [Moet-README] (hybrid section): every token is computed by a few routed experts out of the
// layer's 384.  The score function is not given on the pages; this kernel takes the k largest
// logits (ties to the lower expert id, -0 == +0, descending order) and softmax gates over them.
//
// Each lane holds E/64 logits as 64-bit keys: an order-preserving image of the float in the
// high word and (2^32-1 - expert id) in the low word, so one unsigned max picks the largest
// logit and, among equal logits, the lowest id.  k rounds of a wave max-reduction extract the
// winners; lane j keeps the j-th winner.  Logits are read once, coalesced (lane l reads
// columns l, l+64, ...).
#include "common.h"
#include "kernels.h"

namespace bitmoe {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ gates) {
  const int lane = wave_lane();
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    key[i] = 0;  // below every real key (no logit maps to an all-zero high word)
    if (e < E) key[i] = ((uint64_t)order_key(row[e]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
  }
  uint64_t mine = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      uint64_t o = __shfl_xor(best, off);
      best = o > best ? o : best;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (key[i] == best) key[i] = 0;
    if (lane == j) mine = best;
  }
  const float lg = key_to_float((uint32_t)(mine >> 32));
  const float lmax = __shfl(lg, 0);
  const float z = lane < k ? __expf(lg - lmax) : 0.0f;
  const float sum = wave_sum(z);
  if (lane < k) {
    ids[(size_t)t * k + lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)mine);
    gates[(size_t)t * k + lane] = z / sum;
  }
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
