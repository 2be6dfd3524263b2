// Quantisers: fp32 expert weights -> the packed formats the FFN kernels read.
//
// [Moet-QA] (2-bit expert quantisation on the codebook {-4,-1,1,4}) gives the codebook but
// not how codes and scales are fitted; [Strata-R9700] (the post comparing 3-bit and 2-bit
// experts) judges a quantised expert by how close it stays to the float weights.  The fit
// taken here is the least-squares one of w ~ level[code] * s per 32-weight group, found by
// alternating its two exact half-steps (nearest level for a fixed scale; the scale
// sum(level*w) / sum(level^2) for fixed codes): start at s = max|w| / 4, three rounds, round
// s to bf16 (nearest even), final codes against the stored bf16 scale.  Every decision is
// taken in fp32 in a fixed order (products level*w are exact, sums run k = 0..31, each
// multiply and divide is one IEEE rounding), so the result is deterministic bit for bit.
// Nearest-level rule with t = 2.5 s: code 3 (+4) if w > t, 2 (+1) if 0 <= w <= t, 1 (-1) if
// -t <= w < 0, 0 (-4) if w < -t (ties and -0 go to the smaller magnitude); an all-zero
// group gets scale 0 and code 2.
//
// MXFP4 ([OCP-MX], blocks of 32 along K): shared exponent floor(log2 amax) - 2, clamped to
// the e8m0 range (scale byte 0 for an all-zero block); each element w / 2^shared (exact in
// fp32) rounded to the nearest e2m1 value with ties to the even mantissa, saturating at 6.
//
// One thread per group: the weights are read once (HBM bound: 4 bytes per weight in,
// 0.3125 (2-bit) or 0.53125 (MXFP4) bytes out).
#include "common.h"
#include "kernels.h"

namespace bitmoe {

__device__ __forceinline__ void load32(const float* __restrict__ src, float (&v)[32]) {
  const float4* p = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 q = p[i];
    v[4 * i] = q.x;
    v[4 * i + 1] = q.y;
    v[4 * i + 2] = q.z;
    v[4 * i + 3] = q.w;
  }
}

// code of w for threshold t = 2.5 s (see the rule above): +-4 when |w| > t, the sign from
// w < 0 (so -0 is positive): 2 * !neg + (big != neg)
__device__ __forceinline__ uint32_t w2_code(float w, float t) {
  const uint32_t big = fabsf(w) > t, neg = w < 0.0f;
  return 2u * (neg ^ 1u) + (big ^ neg);
}

__global__ __launch_bounds__(256) void quantize_w2_kernel(const float* __restrict__ w, int64_t groups,
                                                          uint2* __restrict__ codes,
                                                          uint16_t* __restrict__ scales) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= groups) return;
  float v[32];
  load32(w + g * 32, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  float s = amax * 0.25f;  // exact: a power-of-two scaling
  for (int r = 0; r < 3; ++r) {
    const float t = __fmul_rn(2.5f, s);
    // level * w = |level| * |w| (the level takes the sign of w; -0 adds +-0 to a sum that
    // is never -0), and |level| * |w| is exact, so one fma per weight is the same single
    // rounding as the sequential sum; sum(level^2) = 32 + 15 * (number of +-4 codes), exact
    float num = 0.0f;
    int n4 = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float a = fabsf(v[i]);
      const bool big = a > t;
      num = __fmaf_rn(big ? 4.0f : 1.0f, a, num);
      n4 += big ? 1 : 0;
    }
    s = amax > 0.0f ? __fdiv_rn(num, (float)(32 + 15 * n4)) : 0.0f;
  }
  const uint32_t sb = f32_to_bf16_rne(s);
  const float t = __fmul_rn(2.5f, __uint_as_float(sb << 16));
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    lo |= (amax > 0.0f ? w2_code(v[i], t) : 2u) << (2 * i);
    hi |= (amax > 0.0f ? w2_code(v[16 + i], t) : 2u) << (2 * i);
  }
  codes[g] = make_uint2(lo, hi);
  scales[g] = (uint16_t)sb;
}

// nearest e2m1 magnitude index of a >= 0 (saturating at 6), ties to the even index
__device__ __forceinline__ uint32_t e2m1_index(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
         (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
}

__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const float* __restrict__ w, int64_t blocks,
                                                             uint4* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= blocks) return;
  float v[32];
  load32(w + g * 32, v);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // floor(log2 amax) from the fp32 fields (subnormal amax: the position of its top bit)
  const uint32_t ab = __float_as_uint(amax);
  const int ef = (int)(ab >> 23);
  const int fl = ef > 0 ? ef - 127 : (31 - __clz((int)(ab & 0x7FFFFFu))) - 149;
  const int shared = amax > 0.0f ? min(max(fl - 2, -127), 127) : -127;
  // 2^-shared as an fp32 (2^-127 .. 2^127; 2^127 down to 2^-126 normal, 2^-127 subnormal)
  const float inv = shared <= 126 ? __uint_as_float((uint32_t)(127 - shared) << 23) : 0x1p-127f;
  uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float x = v[i] * inv;
    const uint32_t n = e2m1_index(fminf(fabsf(x), 6.0f)) | ((__float_as_uint(v[i]) >> 31) << 3);
    word[i >> 3] |= n << (4 * (i & 7));
  }
  codes[g] = make_uint4(word[0], word[1], word[2], word[3]);
  scales[g] = (uint8_t)(shared + 127);
}

hipError_t launch_quantize_w2(const float* w, int64_t rows, int K, uint32_t* codes, uint16_t* scales,
                              hipStream_t s) {
  const int64_t groups = rows * (K / 32);
  const int64_t grid = (groups + 255) / 256;
  quantize_w2_kernel<<<(unsigned)grid, 256, 0, s>>>(w, groups, reinterpret_cast<uint2*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(const float* w, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s) {
  const int64_t blocks = rows * (K / 32);
  const int64_t grid = (blocks + 255) / 256;
  quantize_mxfp4_kernel<<<(unsigned)grid, 256, 0, s>>>(w, blocks, reinterpret_cast<uint4*>(codes), scales);
  return hipGetLastError();
}

}  // namespace bitmoe
