// Stable grouping of the R = T*k routed rows by expert (a counting sort keyed by expert id).
//
// Rows are split into chunks of kPermuteChunk; each chunk into 8 contiguous wave ranges.
// A wave walks its range 64 rows at a time and ranks equal keys among its lanes with a
// bit-sliced ballot match (lanes with the same expert id), so every row gets
//   position = offsets[e] + rows of e in earlier chunks + rows of e in earlier waves of the
//              chunk + rows of e earlier in the wave,
// which is exactly the stable (expert, token, slot) order.  Integer counts only: the result
// is deterministic.  R <= kPermuteChunk runs as one fused workgroup (one launch, the decode
// case); larger R runs count -> scan -> scatter.
#include "common.h"
#include "kernels.h"
#include "permute_dev.h"

namespace bitmoe {

// One workgroup does everything (R <= kPermuteChunk).
__global__ __launch_bounds__(kPermThreads) void permute_fused(const int32_t* __restrict__ ids,
                                                              int R, int E, int nbits,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ inv) {
  extern __shared__ int32_t smem[];
  permute_block(ids, R, E, nbits, counts, offsets, perm, inv, smem, nullptr);
}

// Multi-chunk path, step 1: per-chunk per-expert counts -> blockhist[chunk][E].
__global__ __launch_bounds__(kPermThreads) void permute_count(const int32_t* __restrict__ ids,
                                                              int R, int E, int nbits,
                                                              int32_t* __restrict__ blockhist) {
  extern __shared__ int32_t smem[];
  int32_t* cnt = smem;
  const int w = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kPermWaves * E; i += kPermThreads) cnt[i] = 0;
  __syncthreads();
  const int c_lo = blockIdx.x * kPermuteChunk, c_hi = min(R, c_lo + kPermuteChunk);
  int lo, hi;
  wave_range(c_lo, c_hi, w, &lo, &hi);
  wave_pass<false>(ids, lo, hi, E, nbits, cnt + w * E, nullptr, nullptr);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    int tot = 0;
    for (int v = 0; v < kPermWaves; ++v) tot += cnt[v * E + e];
    blockhist[(size_t)blockIdx.x * E + e] = tot;
  }
}

// Step 2 (one workgroup): blockhist[c][e] <- rows of e in chunks before c; counts; offsets.
__global__ __launch_bounds__(1024) void permute_scan(int32_t* __restrict__ blockhist, int nchunks,
                                                     int E, int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets) {
  __shared__ int scan_tmp[1024 / kWave + 1];
  int running = 0;
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int e = e0 + threadIdx.x;
    int tot = 0;
    if (e < E)
      for (int c = 0; c < nchunks; ++c) {
        const int v = blockhist[(size_t)c * E + e];
        blockhist[(size_t)c * E + e] = tot;
        tot += v;
      }
    int blk;
    const int ex = block_exclusive_scan<1024>(tot, scan_tmp, &blk);
    if (e < E) {
      counts[e] = tot;
      offsets[e] = running + ex;
    }
    running += blk;
  }
  if (threadIdx.x == 0) offsets[E] = running;
}

// Step 3: positions within each chunk, then the scatter.
__global__ __launch_bounds__(kPermThreads) void permute_scatter(const int32_t* __restrict__ ids,
                                                                int R, int E, int nbits,
                                                                const int32_t* __restrict__ blockhist,
                                                                const int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ perm,
                                                                int32_t* __restrict__ inv) {
  extern __shared__ int32_t smem[];
  int32_t* cnt = smem;
  const int w = threadIdx.x / kWave;
  for (int i = threadIdx.x; i < kPermWaves * E; i += kPermThreads) cnt[i] = 0;
  __syncthreads();
  const int c_lo = blockIdx.x * kPermuteChunk, c_hi = min(R, c_lo + kPermuteChunk);
  int lo, hi;
  wave_range(c_lo, c_hi, w, &lo, &hi);
  wave_pass<false>(ids, lo, hi, E, nbits, cnt + w * E, nullptr, nullptr);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads) {
    int p = offsets[e] + blockhist[(size_t)blockIdx.x * E + e];
    for (int v = 0; v < kPermWaves; ++v) {
      const int c = cnt[v * E + e];
      cnt[v * E + e] = p;
      p += c;
    }
  }
  __syncthreads();
  wave_pass<true>(ids, lo, hi, E, nbits, cnt + w * E, perm, inv);
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_i32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

static int key_bits(int E) {
  int b = 0;
  while ((1 << b) <= E) ++b;  // enough bits to hold the sentinel E
  return b;
}

size_t permute_ws_bytes(int64_t R, int E) {
  if (R <= kPermuteChunk) return 0;
  const int64_t nchunks = (R + kPermuteChunk - 1) / kPermuteChunk;
  return (size_t)(nchunks * E * sizeof(int32_t));
}

hipError_t launch_permute(const int32_t* ids, int R, int E, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, void* ws, hipStream_t s) {
  const int nbits = key_bits(E);
  const size_t lds = (size_t)(kPermWaves * E + kPermThreads / kWave + 1) * sizeof(int32_t);
  if (R <= kPermuteChunk) {
    permute_fused<<<1, kPermThreads, lds, s>>>(ids, R, E, nbits, counts, offsets, perm, inv);
    return hipGetLastError();
  }
  const int nchunks = (R + kPermuteChunk - 1) / kPermuteChunk;
  int32_t* blockhist = (int32_t*)ws;
  permute_count<<<nchunks, kPermThreads, lds, s>>>(ids, R, E, nbits, blockhist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  permute_scan<<<1, 1024, 0, s>>>(blockhist, nchunks, E, counts, offsets);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  permute_scatter<<<nchunks, kPermThreads, lds, s>>>(ids, R, E, nbits, blockhist, offsets, perm,
                                                     inv);
  return hipGetLastError();
}

}  // namespace bitmoe
