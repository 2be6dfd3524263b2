// Host-RAM expert tier: the GPU holds n_slots experts out of E, the rest stay in pinned host
// memory ([Moet-QA], section on what the project teaches: the GPU as a cache of hot experts over
// host RAM, relying on routing locality; [Moet-README], flagship results and launcher: an LRU
// over a slot budget with spare slots).  Three calls: a host-side LRU plan of which experts to
// load into which slots, the asynchronous host -> device copies of those experts, and a kernel
// that maps routed expert ids to slot ids so that the layer runs unchanged on the slot arrays.
#include <hip/hip_runtime.h>

#include <vector>

#include "../../include/bitmoe.h"
#include "kernels.h"

namespace bitmoe {

__global__ __launch_bounds__(256) void remap_kernel(const int32_t* __restrict__ ids, int64_t R,
                                                    const int32_t* __restrict__ slot_of_expert,
                                                    int32_t* __restrict__ slot_ids) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < R) slot_ids[i] = slot_of_expert[ids[i]];
}

}  // namespace bitmoe

using namespace bitmoe;

namespace {

// Packed bytes of one expert's four arrays in format fmt (W2 or W3), matching the layouts of
// moe_weights: W1 has 2I rows of H, W2 has H rows of I.
struct ExpertBytes {
  size_t w1c, w1s, w2c, w2s;
};

bool expert_bytes(const moe_weights* w, ExpertBytes* b) {
  if (!w || w->H <= 0 || w->I <= 0 || w->H % 256 || w->I % 256) return false;
  const size_t n1 = (size_t)2 * w->I * w->H, n2 = (size_t)w->H * w->I;
  if (w->fmt == MOE_FMT_W2) {
    *b = {n1 / 4, n1 / 32 * 2, n2 / 4, n2 / 32 * 2};
  } else if (w->fmt == MOE_FMT_W3) {
    *b = {n1 * 3 / 8, n1 / 64, n2 * 3 / 8, n2 / 64};
  } else {
    return false;
  }
  return true;
}

}  // namespace

extern "C" {

moe_status moe_tier_plan(moe_tier_state* st, const int32_t* ids, int64_t R, int32_t* load_expert,
                         int32_t* load_slot, int32_t* n_load) {
  if (!st || st->E < 1 || st->n_slots < 1 || R < 0 || !n_load) return MOE_ERR_INVALID_ARG;
  if (!st->slot_of_expert || !st->expert_of_slot || !st->last_use) return MOE_ERR_INVALID_ARG;
  if (R > 0 && (!ids || !load_expert || !load_slot)) return MOE_ERR_INVALID_ARG;
  const int E = st->E, S = st->n_slots;
  std::vector<char> need(E, 0);
  for (int64_t i = 0; i < R; ++i) {
    if (ids[i] < 0 || ids[i] >= E) return MOE_ERR_INVALID_ARG;
    need[ids[i]] = 1;
  }
  int n_need = 0;
  for (int e = 0; e < E; ++e) n_need += need[e];
  if (n_need > S) return MOE_ERR_UNSUPPORTED;  // the batch does not fit the slot budget
  const int64_t tick = st->tick + 1;
  // hits: refresh their slots' last use (a slot in use by this batch is never evicted)
  for (int e = 0; e < E; ++e)
    if (need[e] && st->slot_of_expert[e] >= 0) st->last_use[st->slot_of_expert[e]] = tick;
  int nl = 0;
  for (int e = 0; e < E; ++e) {
    if (!need[e] || st->slot_of_expert[e] >= 0) continue;
    // a miss: the lowest empty slot, else the least recently used slot (ties: lowest index);
    // slots used by this batch carry the current tick and are never the minimum while a slot
    // of an earlier batch remains, which n_need <= S guarantees
    int best = -1;
    for (int s = 0; s < S && best < 0; ++s)
      if (st->expert_of_slot[s] < 0) best = s;
    if (best < 0) {
      for (int s = 0; s < S; ++s)
        if (st->last_use[s] < tick && (best < 0 || st->last_use[s] < st->last_use[best])) best = s;
    }
    if (best < 0) return MOE_ERR_UNSUPPORTED;  // unreachable: n_need <= S
    const int old = st->expert_of_slot[best];
    if (old >= 0) st->slot_of_expert[old] = -1;
    st->expert_of_slot[best] = e;
    st->slot_of_expert[e] = best;
    st->last_use[best] = tick;
    load_expert[nl] = e;
    load_slot[nl] = best;
    ++nl;
  }
  st->tick = tick;
  *n_load = nl;
  return MOE_OK;
}

moe_status moe_tier_load(const moe_weights* host_w, const moe_weights* slot_w, const int32_t* load_expert,
                         const int32_t* load_slot, int32_t n_load, void* stream) {
  ExpertBytes b, bs;
  if (!expert_bytes(host_w, &b) || !expert_bytes(slot_w, &bs)) return MOE_ERR_INVALID_ARG;
  if (host_w->fmt != slot_w->fmt || host_w->H != slot_w->H || host_w->I != slot_w->I)
    return MOE_ERR_INVALID_ARG;
  if (n_load < 0) return MOE_ERR_INVALID_ARG;
  if (n_load == 0) return MOE_OK;
  if (!load_expert || !load_slot) return MOE_ERR_INVALID_ARG;
  const void* src[4] = {host_w->w1_codes, host_w->w1_scales, host_w->w2_codes, host_w->w2_scales};
  const void* dst[4] = {slot_w->w1_codes, slot_w->w1_scales, slot_w->w2_codes, slot_w->w2_scales};
  const size_t sz[4] = {b.w1c, b.w1s, b.w2c, b.w2s};
  for (int a = 0; a < 4; ++a)
    if (!src[a] || !dst[a]) return MOE_ERR_INVALID_ARG;
  for (int i = 0; i < n_load; ++i) {
    const int e = load_expert[i], s = load_slot[i];
    if (e < 0 || e >= host_w->E || s < 0 || s >= slot_w->E) return MOE_ERR_INVALID_ARG;
  }
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  for (int i = 0; i < n_load; ++i) {
    const size_t e = (size_t)load_expert[i], s = (size_t)load_slot[i];
    for (int a = 0; a < 4; ++a) {
      const hipError_t err =
          hipMemcpyAsync(const_cast<char*>(static_cast<const char*>(dst[a])) + s * sz[a],
                         static_cast<const char*>(src[a]) + e * sz[a], sz[a], hipMemcpyHostToDevice, hs);
      if (err != hipSuccess) return MOE_ERR_HIP;
    }
  }
  return MOE_OK;
}

moe_status moe_tier_remap(const int32_t* topk_ids, int64_t R, const int32_t* slot_of_expert,
                          int32_t* slot_ids, void* stream) {
  if (R < 0) return MOE_ERR_INVALID_ARG;
  if (R == 0) return MOE_OK;
  if (!topk_ids || !slot_of_expert || !slot_ids) return MOE_ERR_INVALID_ARG;
  const int64_t blocks = (R + 255) / 256;
  if (blocks > 0x7FFFFFFF) return MOE_ERR_INVALID_ARG;
  remap_kernel<<<(unsigned)blocks, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(topk_ids, R, slot_of_expert,
                                                                                   slot_ids);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
