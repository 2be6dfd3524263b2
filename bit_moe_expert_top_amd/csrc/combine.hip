// Gate-weighted combine: out[t] = sum_j gate[t][j] * y_perm[inv[t*k+j]], in fp32, j ascending.
// (The pages do not describe the combine; this is the plain reading of a routed-expert sum.)
// A workgroup per (token, 1024 columns), 16-byte loads of the k expert rows; HBM-bound (R*H*4
// bytes read).
#include "common.h"
#include "kernels.h"

namespace bitmoe {

template <bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ gates, int k,
                                                      int H, void* __restrict__ out) {
  // block (t, column chunk): 256 threads x 4 columns; the expert rows of a token are loaded
  // 8 at a time before they are summed (in slot order), so their loads overlap
  const int t = blockIdx.x;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  if (c >= H / 4) return;
  const int32_t* it = inv + (size_t)t * k;
  const float* gt = gates + (size_t)t * k;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += 8) {
    float4 v[8];
    float g[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + u, k - 1);
      g[u] = gt[j];
      v[u] = reinterpret_cast<const float4*>(y + (size_t)it[j] * H)[c];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + u < k) {
        acc.x = fmaf(g[u], v[u].x, acc.x);
        acc.y = fmaf(g[u], v[u].y, acc.y);
        acc.z = fmaf(g[u], v[u].z, acc.z);
        acc.w = fmaf(g[u], v[u].w, acc.w);
      }
    }
  }
  if (OUT_F32) {
    reinterpret_cast<float4*>((float*)out + (size_t)t * H)[c] = acc;
  } else {
    const uint32_t lo = f32x2_to_bf16x2_rne(acc.x, acc.y);
    const uint32_t hi = f32x2_to_bf16x2_rne(acc.z, acc.w);
    reinterpret_cast<uint2*>((uint16_t*)out + (size_t)t * H)[c] = make_uint2(lo, hi);
  }
}

hipError_t launch_combine(const float* y, const int32_t* inv, const float* w, int T, int k, int H,
                          void* out, bool out_f32, hipStream_t s) {
  const int threads = H / 4 >= 256 ? 256 : 64;
  const dim3 grid(T, (H / 4 + threads - 1) / threads);
  if (out_f32)
    combine_kernel<true><<<grid, threads, 0, s>>>(y, inv, w, k, H, out);
  else
    combine_kernel<false><<<grid, threads, 0, s>>>(y, inv, w, k, H, out);
  return hipGetLastError();
}

}  // namespace bitmoe
