// Top-k routing of one token by one wavefront (device code shared by the routing kernel and
// the fused small-batch front kernel).
//
// [Moet-README] (hybrid section): every token is computed by a few routed experts out of the
// layer's 384.  The score function is not given on the pages; this takes the k largest logits
// (ties to the lower expert id, -0 == +0, descending order) and softmax gates over them.
//
// Each lane holds E/64 logits as 64-bit keys: an order-preserving image of the float in the
// high word and (2^32-1 - expert id) in the low word, so one unsigned max picks the largest
// logit and, among equal logits, the lowest id.  k rounds of a wave max-reduction extract the
// winners; lane j keeps the j-th winner.  Logits are read once, coalesced (lane l reads
// columns l, l+64, ...), all of a lane's loads in flight together.
#pragma once

#include "common.h"

namespace bitmoe {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide maximum of a 64-bit key, the result in every lane.  Within each row of 16 lanes
// four DPP exchanges (xor 1, xor 2, half-row mirror, row mirror) leave the row maximum in every
// lane; the four row maxima are then read as scalars (v_readlane) and combined uniformly.
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max_u64(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max_u64(v, dpp_u64<0x141>(v));  // row_half_mirror
  v = max_u64(v, dpp_u64<0x140>(v));  // row_mirror
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r);
    m = max_u64(m, ((uint64_t)hi << 32) | lo);
  }
  return m;
}

// Route the token whose E logits start at `row` (all 64 lanes of the wave): lane j < k writes
// the j-th expert id and gate to ids[j], gates[j] and, if ids2 is not null, the id to ids2[j].
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int32_t* ids,
                                            float* gates, int32_t* ids2) {
  const int lane = wave_lane();
  // every load is issued before any is used (clamped index, no branch per load)
  float lv[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) lv[i] = row[min(lane + kWave * i, E - 1)];
  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    // 0 is below every real key (no logit maps to an all-zero high word)
    key[i] = e < E ? ((uint64_t)order_key(lv[i]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e) : 0;
  }
  uint64_t mine = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) best = max_u64(best, key[i]);
    best = wave_max_u64(best);
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
    const int32_t id = (int32_t)(0xFFFFFFFFu - (uint32_t)mine);
    ids[lane] = id;
    gates[lane] = z / sum;
    if (ids2) ids2[lane] = id;
  }
}

}  // namespace bitmoe
