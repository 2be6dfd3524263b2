// Stable grouping of routed rows by expert inside one workgroup (device code shared by the
// grouping kernels and the fused small-batch front kernel).  See permute.hip for the method.
#pragma once

#include "common.h"

namespace bitmoe {

constexpr int kPermWaves = 8;
constexpr int kPermThreads = kPermWaves * kWave;

// Lanes of this wave holding the same key (all 64 lanes must be active).
__device__ __forceinline__ uint64_t match_lanes(int key, int nbits) {
  uint64_t m = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    const int bit = (key >> b) & 1;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

// Walk rows [lo, hi) of this wave 64 at a time.  With ASSIGN false, add the wave's per-expert
// counts into cnt[]; with ASSIGN true, cnt[] holds the first position of each expert for this
// wave and the rows are written out.
template <bool ASSIGN>
__device__ __forceinline__ void wave_pass(const int32_t* __restrict__ ids, int lo, int hi, int E,
                                          int nbits, int32_t* cnt, int32_t* __restrict__ perm,
                                          int32_t* __restrict__ inv) {
  const int lane = wave_lane();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int base = lo; base < hi; base += kWave) {
    const int r = base + lane;
    const int key = r < hi ? ids[r] : E;  // E = sentinel for lanes past the end
    const uint64_t m = match_lanes(key, nbits);
    const int rank = __popcll(m & below);
    const int n = __popcll(m);
    if ((unsigned)key < (unsigned)E) {  // ids outside [0, E) are skipped (no LDS access)
      const int start = cnt[key];
      if (ASSIGN) {
        perm[start + rank] = r;
        inv[r] = start + rank;
      }
      if (rank == 0) cnt[key] = start + n;
    }
  }
}

__device__ __forceinline__ void wave_range(int chunk_lo, int chunk_hi, int w, int* lo, int* hi) {
  const int len = chunk_hi - chunk_lo;
  int per = (len + kPermWaves - 1) / kPermWaves;
  per = (per + kWave - 1) / kWave * kWave;
  *lo = min(chunk_hi, chunk_lo + w * per);
  *hi = min(chunk_hi, *lo + per);
}

// R <= 64 rows (a decode batch): wave 0 places them in registers -- a row's position in the
// stable (id, row) order is the number of rows with a smaller id, found bit by bit from the most
// significant one with one ballot per bit, plus the rows with its id on lower lanes -- and every
// thread then counts, for its experts, the ids below and equal to it among the <= 64 kept in LDS.
// No per-wave counters, no scans; the outputs are those of the general path (ids outside [0, E)
// skipped).  keys: 64 ints of LDS.
__device__ __forceinline__ void permute_small(const int32_t* ids, int R, int E, int nbits,
                                              int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                              int32_t* keys, int32_t* off2) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int id = lane < R ? ids[lane] : E;
    const bool ok = (unsigned)id < (unsigned)E;
    const int key = ok ? id : E;  // E (the sentinel) sorts after every id and is never counted
    keys[lane] = key;
    const uint64_t cand = __ballot(ok);
    uint64_t same = cand;  // rows whose id agrees with this row's above bit b
    int below = 0;         // rows with a smaller id
    for (int b = nbits - 1; b >= 0; --b) {
      const int bit = (key >> b) & 1;
      const uint64_t bal = __ballot(bit) & cand;
      if (bit) below += __popcll(same & ~bal);
      same &= bit ? bal : ~bal;
    }
    if (ok) {
      const int pos = below + __popcll(same & ((1ull << lane) - 1ull));
      perm[pos] = lane;
      inv[lane] = pos;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += kPermThreads) {
    int lt = 0, eq = 0;
    for (int r = 0; r < R; ++r) {
      const int k = keys[r];
      lt += k < e;
      eq += k == e;
    }
    if (e < E) counts[e] = eq;
    offsets[e] = lt;
    if (off2) off2[e] = lt;
  }
}

// Group R <= kPermuteChunk rows in one workgroup of kPermThreads threads: counts[E],
// offsets[E+1], perm[R], inv[R] (global), and the offsets also into off2 if not null.
// smem: kPermWaves * E + kPermThreads / 64 + 1 ints.
__device__ __forceinline__ void permute_block(const int32_t* ids, int R, int E, int nbits,
                                              int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                              int32_t* smem, int32_t* off2) {
  if (R <= kWave) {
    permute_small(ids, R, E, nbits, counts, offsets, perm, inv, smem, off2);
    return;
  }
  int32_t* cnt = smem;                        // [kPermWaves][E]
  int32_t* scan_tmp = smem + kPermWaves * E;  // kPermThreads/64 + 1
  const int w = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kPermWaves * E; i += kPermThreads) cnt[i] = 0;
  __syncthreads();
  int lo, hi;
  wave_range(0, R, w, &lo, &hi);
  wave_pass<false>(ids, lo, hi, E, nbits, cnt + w * E, perm, inv);
  __syncthreads();
  // totals per expert, exclusive scan over experts, first position per (wave, expert)
  int running = 0;
  for (int e0 = 0; e0 < E; e0 += kPermThreads) {
    const int e = e0 + threadIdx.x;
    int tot = 0;
    if (e < E)
      for (int v = 0; v < kPermWaves; ++v) tot += cnt[v * E + e];
    int blk;
    const int ex = block_exclusive_scan<kPermThreads>(tot, scan_tmp, &blk);
    if (e < E) {
      counts[e] = tot;
      offsets[e] = running + ex;
      if (off2) off2[e] = running + ex;
      int p = running + ex;
      for (int v = 0; v < kPermWaves; ++v) {
        const int c = cnt[v * E + e];
        cnt[v * E + e] = p;
        p += c;
      }
    }
    running += blk;
  }
  if (threadIdx.x == 0) {
    offsets[E] = running;
    if (off2) off2[E] = running;
  }
  __syncthreads();
  wave_pass<true>(ids, lo, hi, E, nbits, cnt + w * E, perm, inv);
}

}  // namespace bitmoe
