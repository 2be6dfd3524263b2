// The FFN work list, built on the device from the grouping offsets (no host round trip).
#pragma once

#include "common.h"

namespace bitmoe {

// Run by one block of 1024 threads.  plan[0] = number of items; then int4 items
// {expert, first grouped row, rows, hot slot or -1}: the rows of every expert of the
// requested kind (low-bit experts, or hot experts if want_hot) split into items of at most
// `chunk` rows, experts in id order.
__device__ __forceinline__ void build_plan(const int32_t* __restrict__ offsets, int E, int chunk,
                                           const int32_t* __restrict__ hot_ids, int n_hot, int want_hot,
                                           int32_t* __restrict__ plan) {
  __shared__ int scan_tmp[1024 / kWave + 1];
  __shared__ int16_t slot_of[1024];
  for (int e = threadIdx.x; e < E; e += 1024) slot_of[e] = -1;
  __syncthreads();
  for (int s = threadIdx.x; s < n_hot; s += 1024) {
    const int he = hot_ids[s];
    if ((unsigned)he < (unsigned)E) slot_of[he] = (int16_t)s;  // ids outside [0, E) are ignored
  }
  __syncthreads();
  int4* items = reinterpret_cast<int4*>(plan + 4);
  int running = 0;
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int e = e0 + threadIdx.x;
    int cnt = 0, slot = -1;
    if (e < E) {
      slot = slot_of[e];
      cnt = offsets[e + 1] - offsets[e];
      if ((slot >= 0) != (want_hot != 0)) cnt = 0;
    }
    const int nch = (cnt + chunk - 1) / chunk;
    int tot;
    const int ex = block_exclusive_scan<1024>(nch, scan_tmp, &tot);
    for (int c = 0; c < nch; ++c)
      items[running + ex + c] = make_int4(e, offsets[e] + c * chunk, min(chunk, cnt - c * chunk), slot);
    running += tot;
  }
  if (threadIdx.x == 0) plan[0] = running;
}

}  // namespace bitmoe

namespace bitmoe {

// Two work lists (one block of NT threads), for batches that use both FFN kernels: a low-bit
// expert with more than `small_max` rows goes to the grouped-GEMM list in items of at most
// `gemm_chunk` rows; one with fewer goes to the streaming list in items of at most `small_max`
// rows.  With gemm_enabled == 0 every expert goes to the streaming list.  Hot experts are left
// out, unless hot_residual: then they go to the streaming list at any size, each item carrying
// the expert's hot slot (the FP4 residual the streaming kernel adds).  Both lists have the
// layout of build_plan.  The GEMM list holds an expert's short last item (at most
// gemm_chunk / 2 rows, which the GEMM runs on half its matrix tiles) after all the full items:
// the GEMM pairs consecutive items on the same weight tiles, and a pair of unequal length
// would leave its two workgroups out of step, each fetching the tiles on its own.
template <int NT = 1024>
__device__ __forceinline__ void build_plan2(const int32_t* __restrict__ offsets, int E, int small_max,
                                            int gemm_chunk, int gemm_enabled,
                                            const int32_t* __restrict__ hot_ids, int n_hot, int hot_residual,
                                            int32_t* __restrict__ plan_s, int32_t* __restrict__ plan_g) {
  __shared__ int scan_tmp[NT / kWave + 1];
  __shared__ int16_t slot_of[1024];  // E <= 1024
  for (int e = threadIdx.x; e < E; e += NT) slot_of[e] = -1;
  __syncthreads();
  for (int s = threadIdx.x; s < n_hot; s += NT) {
    const int he = hot_ids[s];
    if ((unsigned)he < (unsigned)E) slot_of[he] = (int16_t)s;  // ids outside [0, E) are ignored
  }
  __syncthreads();
  int4* items_s = reinterpret_cast<int4*>(plan_s + 4);
  int4* items_g = reinterpret_cast<int4*>(plan_g + 4);
  // per expert: its rows, its list, its item count, and (GEMM list) whether its last item is short
  auto expert_items = [&](int e, int& cnt, int& slot, bool& big, int& chunk, int& nch, int& shrt) {
    cnt = 0;
    slot = -1;
    if (e < E) {
      slot = slot_of[e];
      if (slot < 0 || hot_residual) cnt = offsets[e + 1] - offsets[e];
    }
    big = gemm_enabled && cnt > small_max && slot < 0;
    chunk = big ? gemm_chunk : small_max;
    nch = (cnt + chunk - 1) / chunk;
    shrt = big && 2 * (cnt - (nch - 1) * chunk) <= gemm_chunk ? 1 : 0;
  };
  int run_s = 0, run_g = 0;
  for (int e0 = 0; e0 < E; e0 += NT) {
    const int e = e0 + threadIdx.x;
    int cnt, slot, chunk, nch, shrt;
    bool big;
    expert_items(e, cnt, slot, big, chunk, nch, shrt);
    const int nfull = nch - shrt;  // items written in this pass
    int tot_s, tot_g;
    const int ex_s = block_exclusive_scan<NT>(big ? 0 : nch, scan_tmp, &tot_s);
    const int ex_g = block_exclusive_scan<NT>(big ? nfull : 0, scan_tmp, &tot_g);
    int4* dst = big ? items_g + run_g + ex_g : items_s + run_s + ex_s;
    for (int c = 0; c < nfull; ++c) dst[c] = make_int4(e, offsets[e] + c * chunk, min(chunk, cnt - c * chunk), slot);
    run_s += tot_s;
    run_g += tot_g;
  }
  // second pass: the short last items of the GEMM list, after every full one
  for (int e0 = 0; gemm_enabled && e0 < E; e0 += NT) {
    const int e = e0 + threadIdx.x;
    int cnt, slot, chunk, nch, shrt;
    bool big;
    expert_items(e, cnt, slot, big, chunk, nch, shrt);
    int tot_h;
    const int ex_h = block_exclusive_scan<NT>(shrt, scan_tmp, &tot_h);
    if (shrt) items_g[run_g + ex_h] = make_int4(e, offsets[e] + (nch - 1) * chunk, cnt - (nch - 1) * chunk, slot);
    run_g += tot_h;
  }
  if (threadIdx.x == 0) {
    plan_s[0] = run_s;
    plan_g[0] = run_g;
  }
}

}  // namespace bitmoe
