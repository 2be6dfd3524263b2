// Expert FFN over low-bit codebook weights: weight-streaming kernels with MFMA on 16-token
// tiles (the decode shape: few tokens per expert, every weight byte read once).
//
// [Moet-QA] (2-bit experts): weights are 2-bit codes on the sign-symmetric codebook
// {-4,-1,1,4} with a bf16 scale per group of 32 along K.  [Moet-README] release notes of
// -r23: each expert is FC1 (gate and up projections), SwiGLU, then FC2.
//
// Work split.  A task is (chunk of <= 16*NT grouped rows of one expert, 32 weight rows);
// a workgroup of 4 waves takes a task and splits K in four.  Each wave streams its rows'
// packed codes with 16-byte loads (64 codes per lane per step), decodes them to bf16 in
// registers and feeds v_mfma_f32_16x16x32_bf16 with the weights as A (16 rows x 32 k) and
// the tokens as B (32 k x 16 tokens).  The four K-partials are summed in LDS in a fixed
// order (deterministic), then FC1 applies SwiGLU and stores h (bf16), FC2 stores y (fp32).
//
// Decoding 2-bit codes to bf16.  The four levels are +-1 and +-4, so level*scale is the
// scale's bf16 with the sign flipped and/or 2 added to the exponent: exact, and the low
// byte of the bf16 is the scale's low byte for all four codes.  Per 32-weight group a lane
// builds a byte table {hi byte of -4s, -s, s, 4s | lo byte of s}; one v_perm_b32 then turns
// a selector holding two codes into two bf16 weights.  The selector needs the two codes in
// bytes 1 and 3; from one 32-bit word (codes 0..15) the cheap pairs are (4+m, 12+m), taken
// with a right shift by 2m, and (m, 8+m), taken with a left shift by 8-2m.  MFMA only needs
// A and B to agree on which k sits in which slot, so within every 16 consecutive k the
// k-slots are ordered  4,12,5,13,6,14,7,15, 0,8,1,9,2,10,3,11  on both sides: the token
// operand is stored in that order (x by a small permute kernel, h by FC1's epilogue).
// About 1.5 VALU operations per weight, below the ~2.2 the HBM rate allows at 70 %.
#include "common.h"
#include "kernels.h"

namespace bitmoe {

// ------------------------------------------------------------------ 2-bit decoding
// Byte table of one group: lo = {hi(-4s), hi(-s), hi(s), hi(4s)}, hi byte 0 = lo byte of s.
__device__ __forceinline__ void w2_table(uint32_t s16, uint32_t& lo, uint32_t& hi) {
  const uint32_t hb = (s16 >> 8) & 0xFFu;
  lo = ((hb * 0x01010101u) ^ 0x00008080u) + 0x01000001u;
  hi = s16 & 0xFFu;
}

// Four bf16 pairs (one MFMA operand) from one code word.  HALF 0: pairs (4+m, 12+m);
// HALF 1: pairs (m, 8+m), m = 0..3; the first code of a pair is the low bf16.
template <int HALF>
__device__ __forceinline__ u32x4 w2_decode(uint32_t w, uint32_t lo, uint32_t hi) {
  constexpr uint32_t M = 0x03000300u, C = 0x00040004u;  // codes in bytes 1, 3; selector 4 in bytes 0, 2
  u32x4 r;
  if (HALF == 0) {
    r[0] = byte_perm(hi, lo, (w & M) | C);
    r[1] = byte_perm(hi, lo, ((w >> 2) & M) | C);
    r[2] = byte_perm(hi, lo, ((w >> 4) & M) | C);
    r[3] = byte_perm(hi, lo, ((w >> 6) & M) | C);
  } else {
    r[0] = byte_perm(hi, lo, ((w << 8) & M) | C);
    r[1] = byte_perm(hi, lo, ((w << 6) & M) | C);
    r[2] = byte_perm(hi, lo, ((w << 4) & M) | C);
    r[3] = byte_perm(hi, lo, ((w << 2) & M) | C);
  }
  return r;
}

// Slot of k = f (0..15) inside 16 consecutive k, for the order 4,12,5,13,6,14,7,15,0,8,1,9,2,10,3,11.
__device__ __forceinline__ int kpos16(int f) {
  // f = 4q + i  ->  2i + 8*(1 - (q & 1)) + (q >> 1)
  const int q = f >> 2, i = f & 3;
  return 2 * i + ((q & 1) ^ 1) * 8 + (q >> 1);
}

// ------------------------------------------------------------------ work list
size_t plan_bytes(int64_t max_items) { return (size_t)(16 + 16 * max_items); }

// Block 0 builds the work list; blocks 1.. store x in the k-slot order of the MFMA operand.
//   work list: plan[0] = number of items, then int4 items {expert, first row, rows, hot slot}:
//   the grouped rows of every expert (low-bit experts, or hot experts if want_hot), split
//   into items of at most `chunk` rows, experts in id order.
//   xp[t][16c + p] = x[t][16c + s(p)], s = 4,12,5,13,6,14,7,15,0,8,1,9,2,10,3,11.
__global__ __launch_bounds__(1024) void prepare_kernel(const int32_t* __restrict__ offsets, int E,
                                                       int chunk, const int32_t* __restrict__ hot_ids,
                                                       int n_hot, int want_hot,
                                                       int32_t* __restrict__ plan,
                                                       const uint4* __restrict__ x, int nchunks,
                                                       uint4* __restrict__ xp) {
  if (blockIdx.x > 0) {
    const int c = (blockIdx.x - 1) * 1024 + threadIdx.x;
    if (c >= nchunks) return;
    const uint4 a = x[2 * c], b = x[2 * c + 1];  // dwords d0..d3 = a, d4..d7 = b
    uint4 o0, o1;
    o0.x = byte_perm(b.z, a.z, 0x05040100u);  // (x4, x12)
    o0.y = byte_perm(b.z, a.z, 0x07060302u);  // (x5, x13)
    o0.z = byte_perm(b.w, a.w, 0x05040100u);  // (x6, x14)
    o0.w = byte_perm(b.w, a.w, 0x07060302u);  // (x7, x15)
    o1.x = byte_perm(b.x, a.x, 0x05040100u);  // (x0, x8)
    o1.y = byte_perm(b.x, a.x, 0x07060302u);  // (x1, x9)
    o1.z = byte_perm(b.y, a.y, 0x05040100u);  // (x2, x10)
    o1.w = byte_perm(b.y, a.y, 0x07060302u);  // (x3, x11)
    xp[2 * c] = o0;
    xp[2 * c + 1] = o1;
    return;
  }
  __shared__ int scan_tmp[1024 / kWave + 1];
  __shared__ int16_t slot_of[1024];
  for (int e = threadIdx.x; e < E; e += 1024) slot_of[e] = -1;
  __syncthreads();
  for (int s = threadIdx.x; s < n_hot; s += 1024) slot_of[hot_ids[s]] = (int16_t)s;
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

hipError_t launch_prepare(const int32_t* offsets, int E, int chunk_rows, const int32_t* hot_ids,
                          int n_hot, bool want_hot, int32_t* plan, const uint16_t* x, int T, int H,
                          uint16_t* xp, hipStream_t s) {
  const int nchunks = xp ? T * (H / 16) : 0;
  const int blocks = 1 + (nchunks + 1023) / 1024;
  prepare_kernel<<<blocks, 1024, 0, s>>>(offsets, E, chunk_rows, hot_ids, n_hot, want_hot ? 1 : 0,
                                         plan, (const uint4*)x, nchunks, (uint4*)xp);
  return hipGetLastError();
}

// ------------------------------------------------------------------ the streaming kernel
__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// FC == 1: A rows = gate rows 16cb+i and up rows I+16cb+i of W1 (K = H), epilogue SwiGLU -> h.
// FC == 2: A rows = rows 32cb+i and 32cb+16+i of W2 (K = I), epilogue -> y (fp32).
template <int FC, int NT>
__global__ __launch_bounds__(256) void w2_stream_kernel(
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales, int rows_per_expert,
    int K, int width, int ktop, const uint16_t* __restrict__ bsrc, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ plan, void* __restrict__ out) {
  __shared__ f32x4 red[4][2 * NT][kWave];
  const int lane = wave_lane(), w = threadIdx.x / kWave;
  const int i16 = lane & 15, q = lane >> 4;
  const int n_items = plan[0];
  const int4* items = reinterpret_cast<const int4*>(plan + 4);
  const int ncb = FC == 1 ? width / 16 : rows_per_expert / 32;
  const int total = n_items * ncb;
  // wave w takes 256-wide K steps [it_lo, it_hi) of the K/256 steps (K % 256 == 0)
  const int n_all = K / 256;
  const int it_lo = (w * n_all) / 4, it_hi = ((w + 1) * n_all) / 4;
  const int n_it = it_hi - it_lo;
  const int wpr = K / 16, spr = K / 32;
  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    const int item = task / ncb, cb = task - item * ncb;
    const int4 itm = items[item];
    const int e = itm.x, r0 = itm.y, nrows = itm.z;
    const int rowA0 = FC == 1 ? 16 * cb + i16 : 32 * cb + i16;
    const int rowA1 = FC == 1 ? width + 16 * cb + i16 : 32 * cb + 16 + i16;
    const size_t ebase = (size_t)e * rows_per_expert;
    const int k0 = 256 * it_lo;
    const uint32_t* c0 = codes + (ebase + rowA0) * wpr + k0 / 16 + 4 * q;
    const uint32_t* c1 = codes + (ebase + rowA1) * wpr + k0 / 16 + 4 * q;
    const uint32_t* s0 = reinterpret_cast<const uint32_t*>(scales + (ebase + rowA0) * spr + k0 / 32 + 2 * q);
    const uint32_t* s1 = reinterpret_cast<const uint32_t*>(scales + (ebase + rowA1) * spr + k0 / 32 + 2 * q);
    const uint16_t* brow[NT];
    bool bval[NT];
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) {
      const int n = 16 * bt + i16;
      bval[bt] = n < nrows;
      size_t rowb = 0;
      if (bval[bt]) rowb = FC == 1 ? (size_t)(perm[r0 + n] / ktop) : (size_t)(r0 + n);
      brow[bt] = bsrc + rowb * K + k0 + 64 * q;
    }
    f32x4 acc0[NT], acc1[NT];
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) {
      acc0[bt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[bt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    u32x4 cw0 = u32x4{0u, 0u, 0u, 0u}, cw1 = cw0;
    uint32_t sw0 = 0, sw1 = 0;
    if (n_it > 0) {
      cw0 = load16(c0);
      cw1 = load16(c1);
      sw0 = s0[0];
      sw1 = s1[0];
    }
    for (int it = 0; it < n_it; ++it) {
      u32x4 nw0 = cw0, nw1 = cw1;
      uint32_t ns0 = sw0, ns1 = sw1;
      if (it + 1 < n_it) {
        nw0 = load16(c0 + 16 * (it + 1));
        nw1 = load16(c1 + 16 * (it + 1));
        ns0 = s0[4 * (it + 1)];
        ns1 = s1[4 * (it + 1)];
      }
      uint32_t t0lo[2], t0hi[2], t1lo[2], t1hi[2];
      w2_table(sw0 & 0xFFFFu, t0lo[0], t0hi[0]);
      w2_table(sw0 >> 16, t0lo[1], t0hi[1]);
      w2_table(sw1 & 0xFFFFu, t1lo[0], t1hi[0]);
      w2_table(sw1 >> 16, t1lo[1], t1hi[1]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 b[NT][2];
#pragma unroll
        for (int bt = 0; bt < NT; ++bt) {
          if (bval[bt]) {
            b[bt][0] = load16(brow[bt] + 256 * it + 16 * j);
            b[bt][1] = load16(brow[bt] + 256 * it + 16 * j + 8);
          } else {
            b[bt][0] = u32x4{0u, 0u, 0u, 0u};
            b[bt][1] = u32x4{0u, 0u, 0u, 0u};
          }
        }
        const int g = j >> 1;
        {
          const u32x4 a0 = w2_decode<0>(cw0[j], t0lo[g], t0hi[g]);
          const u32x4 a1 = w2_decode<0>(cw1[j], t1lo[g], t1hi[g]);
#pragma unroll
          for (int bt = 0; bt < NT; ++bt) {
            acc0[bt] = mfma_16x16x32_bf16(a0, b[bt][0], acc0[bt]);
            acc1[bt] = mfma_16x16x32_bf16(a1, b[bt][0], acc1[bt]);
          }
        }
        {
          const u32x4 a0 = w2_decode<1>(cw0[j], t0lo[g], t0hi[g]);
          const u32x4 a1 = w2_decode<1>(cw1[j], t1lo[g], t1hi[g]);
#pragma unroll
          for (int bt = 0; bt < NT; ++bt) {
            acc0[bt] = mfma_16x16x32_bf16(a0, b[bt][1], acc0[bt]);
            acc1[bt] = mfma_16x16x32_bf16(a1, b[bt][1], acc1[bt]);
          }
        }
      }
      cw0 = nw0;
      cw1 = nw1;
      sw0 = ns0;
      sw1 = ns1;
    }
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) {
      red[w][bt][lane] = acc0[bt];
      red[w][NT + bt][lane] = acc1[bt];
    }
    __syncthreads();
    if (w < NT) {
      const int bt = w;
      const f32x4 a = ((red[0][bt][lane] + red[1][bt][lane]) + red[2][bt][lane]) + red[3][bt][lane];
      const f32x4 b = ((red[0][NT + bt][lane] + red[1][NT + bt][lane]) + red[2][NT + bt][lane]) +
                      red[3][NT + bt][lane];
      const int n = 16 * bt + i16;
      if (n < nrows) {
        const size_t r = (size_t)(r0 + n);
        if (FC == 1) {
          uint16_t* h = reinterpret_cast<uint16_t*>(out) + r * width + 16 * cb;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gt = a[i], up = b[i];
            const float hv = gt / (1.0f + __expf(-gt)) * up;
            h[kpos16(4 * q + i)] = (uint16_t)f32_to_bf16_rne(hv);
          }
        } else {
          float* y = reinterpret_cast<float*>(out) + r * width + 32 * cb + 4 * q;
          *reinterpret_cast<f32x4*>(y) = a;
          *reinterpret_cast<f32x4*>(y + 16) = b;
        }
      }
    }
    __syncthreads();
  }
}

static int grid_for(int64_t tasks) {
  const int64_t cap = 256 * 8;
  return (int)(tasks < cap ? (tasks > 0 ? tasks : 1) : cap);
}

template <int FC>
static hipError_t launch_w2(const uint32_t* codes, const uint16_t* scales, int rows, int K,
                            int width, int ktop, const uint16_t* bsrc, const int32_t* perm,
                            const int32_t* plan, int64_t tasks, int nt, void* out, hipStream_t s) {
  const int grid = grid_for(tasks);
  if (nt == 1)
    w2_stream_kernel<FC, 1><<<grid, 256, 0, s>>>(codes, scales, rows, K, width, ktop, bsrc, perm, plan, out);
  else if (nt == 2)
    w2_stream_kernel<FC, 2><<<grid, 256, 0, s>>>(codes, scales, rows, K, width, ktop, bsrc, perm, plan, out);
  else
    w2_stream_kernel<FC, 4><<<grid, 256, 0, s>>>(codes, scales, rows, K, width, ktop, bsrc, perm, plan, out);
  return hipGetLastError();
}

hipError_t launch_lowbit_fc1(const LowbitWeights& w, int E, int H, int I, int k,
                             const uint16_t* xp, const int32_t* perm, const int32_t* plan,
                             int max_items, int nt, uint16_t* hbuf, hipStream_t s) {
  (void)E;
  if (w.fmt != 1) return hipErrorInvalidValue;
  return launch_w2<1>((const uint32_t*)w.w1_codes, (const uint16_t*)w.w1_scales, 2 * I, H, I, k,
                      xp, perm, plan, (int64_t)max_items * (I / 16), nt, hbuf, s);
}

hipError_t launch_lowbit_fc2(const LowbitWeights& w, int E, int H, int I,
                             const uint16_t* hbuf, const int32_t* plan, int max_items, int nt,
                             float* y, hipStream_t s) {
  (void)E;
  if (w.fmt != 1) return hipErrorInvalidValue;
  return launch_w2<2>((const uint32_t*)w.w2_codes, (const uint16_t*)w.w2_scales, H, I, H, 1, hbuf,
                      nullptr, plan, (int64_t)max_items * (H / 32), nt, y, s);
}

// ------------------------------------------------------------------ debug decode
// One thread per code word: decode with the kernels' own table/perm path, write natural order.
__global__ __launch_bounds__(256) void w2_debug_kernel(const uint32_t* __restrict__ codes,
                                                       const uint16_t* __restrict__ scales,
                                                       int64_t nwords, int K,
                                                       float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nwords) return;
  const int wpr = K / 16;
  const int64_t row = i / wpr;
  const int wc = (int)(i - row * wpr);
  const uint32_t s16 = scales[row * (K / 32) + wc / 2];
  uint32_t lo, hi;
  w2_table(s16, lo, hi);
  const uint32_t wd = codes[i];
  const u32x4 p0 = w2_decode<0>(wd, lo, hi), p1 = w2_decode<1>(wd, lo, hi);
  float* o = out + row * K + 16 * wc;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    o[4 + m] = bf16_to_f32(p0[m] & 0xFFFFu);
    o[12 + m] = bf16_to_f32(p0[m] >> 16);
    o[m] = bf16_to_f32(p1[m] & 0xFFFFu);
    o[8 + m] = bf16_to_f32(p1[m] >> 16);
  }
}

hipError_t launch_debug_dequant(const LowbitWeights& w, int E, int H, int I, int e, int which,
                                float* out, hipStream_t s) {
  (void)E;
  const int rows = which == 1 ? 2 * I : H;
  const int K = which == 1 ? H : I;
  if (w.fmt != 1) return hipErrorInvalidValue;
  const uint32_t* codes = (const uint32_t*)(which == 1 ? w.w1_codes : w.w2_codes) + (size_t)e * rows * (K / 16);
  const uint16_t* scales = (const uint16_t*)(which == 1 ? w.w1_scales : w.w2_scales) + (size_t)e * rows * (K / 32);
  const int64_t nwords = (int64_t)rows * (K / 16);
  w2_debug_kernel<<<(unsigned)((nwords + 255) / 256), 256, 0, s>>>(codes, scales, nwords, K, out);
  return hipGetLastError();
}

}  // namespace bitmoe
