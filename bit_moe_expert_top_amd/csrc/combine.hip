// Gate-weighted combine: out[t] = sum_j gate[t][j] * y_perm[inv[t*k+j]], in fp32, j ascending.
// (The pages do not describe the combine; this is the plain reading of a routed-expert sum.)
// One workgroup per token, 16-byte loads of the k expert rows; HBM-bound (R*H*4 bytes read).
#include "common.h"
#include "kernels.h"

namespace bitmoe {

template <bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ gates, int k,
                                                      int H, void* __restrict__ out) {
  const int t = blockIdx.x;
  const int32_t* it = inv + (size_t)t * k;
  const float* gt = gates + (size_t)t * k;
  for (int c = threadIdx.x; c < H / 4; c += blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float g = gt[j];
      const float4 v = reinterpret_cast<const float4*>(y + (size_t)it[j] * H)[c];
      acc.x = fmaf(g, v.x, acc.x);
      acc.y = fmaf(g, v.y, acc.y);
      acc.z = fmaf(g, v.z, acc.z);
      acc.w = fmaf(g, v.w, acc.w);
    }
    if (OUT_F32) {
      reinterpret_cast<float4*>((float*)out + (size_t)t * H)[c] = acc;
    } else {
      const uint32_t lo = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
      const uint32_t hi = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
      reinterpret_cast<uint2*>((uint16_t*)out + (size_t)t * H)[c] = make_uint2(lo, hi);
    }
  }
}

hipError_t launch_combine(const float* y, const int32_t* inv, const float* w, int T, int k, int H,
                          void* out, bool out_f32, hipStream_t s) {
  const int threads = H / 4 >= 256 ? 256 : 64;
  if (out_f32)
    combine_kernel<true><<<T, threads, 0, s>>>(y, inv, w, k, H, out);
  else
    combine_kernel<false><<<T, threads, 0, s>>>(y, inv, w, k, H, out);
  return hipGetLastError();
}

}  // namespace bitmoe
