// The front of a decode-sized layer: routing, grouping and the low-bit FFN's preparation (its
// work lists, x in the k-slot order), for R = T*k <= kPermuteChunk rows.
//
// A decode step is a chain of short kernels whose fixed start and drain costs add up ([Moet-README]
// README tables: the decode step is graph-captured); here block 0 routes the T tokens (one wave
// per token, route_dev.h), groups the R rows (permute_dev.h) and builds the work lists (plan.h)
// from the offsets it keeps in LDS, while the other blocks store x in slot order.  Above
// kFrontOneLaunchT tokens the routing would keep block 0 busy for longer than a launch costs,
// so the route kernel runs first (one wave per token over the whole GPU) and block 0 reads its
// ids.  The outputs are those of moe_route, moe_permute and stage 0 of moe_expert_ffn, bit for bit.
#include "common.h"
#include "kernels.h"
#include "lowbit_fmt.h"
#include "permute_dev.h"
#include "plan.h"
#include "route_dev.h"

namespace bitmoe {

template <int VPL, bool ROUTE>
__global__ __launch_bounds__(kPermThreads) void front_kernel(FrontArgs a) {
  if (blockIdx.x > 0) {
    const int c = (blockIdx.x - 1) * kPermThreads + threadIdx.x;
    if (c < a.nchunks) x_chunk_to_slots(a.x, c, a.fmt, a.xp);
    return;
  }
  extern __shared__ int32_t smem[];
  const int R = a.T * a.k;
  int32_t* ids_l = smem;                // [R]: the routed ids, row t*k + j
  int32_t* off_l = ids_l + R;           // [E + 1]: the grouping offsets
  int32_t* group_smem = off_l + a.E + 1;  // permute_block's scratch
  if (ROUTE) {
    const int w = threadIdx.x / kWave;
    for (int t = w; t < a.T; t += kPermWaves)
      route_token<VPL>(a.logits + (size_t)t * a.E, a.E, a.k, a.ids + t * a.k, a.gates + t * a.k, ids_l + t * a.k);
  } else {  // routed by the route kernel, launched just before on the same stream
    for (int i = threadIdx.x; i < R; i += kPermThreads) ids_l[i] = a.ids[i];
  }
  __syncthreads();
  permute_block(ids_l, R, a.E, a.nbits, a.counts, a.offsets, a.perm, a.inv, group_smem, off_l);
  __syncthreads();
  build_plan2<kPermThreads>(off_l, a.E, a.small_max, a.gemm_chunk, a.gemm_enabled, a.hot_ids, a.n_hot,
                            a.hot_residual, a.plan_s, a.plan_g);
}

size_t front_lds_bytes(int T, int E, int k) {
  return (size_t)(T * k + E + 1 + kPermWaves * E + kPermThreads / kWave + 1) * sizeof(int32_t);
}

hipError_t launch_front(const FrontArgs& a, int H, hipStream_t s) {
  const int per = a.fmt == W2Fmt::kId ? 16 : 32;  // k per thread of the slot-order copy
  FrontArgs b = a;
  b.nchunks = a.T * (H / per);
  int nb = 0;
  while ((1 << nb) <= a.E) ++nb;  // enough bits to hold the sentinel E
  b.nbits = nb;
  const int blocks = 1 + (b.nchunks + kPermThreads - 1) / kPermThreads;
  const size_t lds = front_lds_bytes(a.T, a.E, a.k);
  if (a.T > kFrontOneLaunchT) {
    const hipError_t e = launch_route(a.logits, a.T, a.E, a.k, a.ids, a.gates, s);
    if (e != hipSuccess) return e;
    front_kernel<1, false><<<blocks, kPermThreads, lds, s>>>(b);
    return hipGetLastError();
  }
  const int vpl = (a.E + kWave - 1) / kWave;
  if (vpl <= 1) front_kernel<1, true><<<blocks, kPermThreads, lds, s>>>(b);
  else if (vpl <= 2) front_kernel<2, true><<<blocks, kPermThreads, lds, s>>>(b);
  else if (vpl <= 4) front_kernel<4, true><<<blocks, kPermThreads, lds, s>>>(b);
  else if (vpl <= 6) front_kernel<6, true><<<blocks, kPermThreads, lds, s>>>(b);
  else if (vpl <= 8) front_kernel<8, true><<<blocks, kPermThreads, lds, s>>>(b);
  else front_kernel<16, true><<<blocks, kPermThreads, lds, s>>>(b);
  return hipGetLastError();
}

}  // namespace bitmoe
