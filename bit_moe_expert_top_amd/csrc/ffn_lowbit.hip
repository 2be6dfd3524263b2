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
// scale's bf16 with the sign flipped and/or 2 added to the exponent: exact, and every
// decoded weight of a group has the scale's low byte.  Per 32-weight group a lane keeps a
// byte table of the four high bytes {-4s, -s, s, 4s}.  For one 32-bit word (codes 0..15):
// mask the word (shifted by 2s) with 0x03030303, which leaves codes s, 4+s, 8+s, 12+s one
// per byte -- a v_perm_b32 selector -- look their high bytes up with one v_perm_b32, and
// interleave them with the low byte by two more: two bf16 pairs per 2.4 VALU operations,
// ~1.2 per weight, under the ~1.5 that the HBM rate leaves per weight at peak.  MFMA only
// needs A and B to agree on which k sits in which slot, so within every 16 consecutive k the
// slots hold k = 0,4,8,12, 1,5,9,13, 2,6,10,14, 3,7,11,15 (a 4x4 transpose) on both sides:
// the token operand is stored in that order (x by the prepare kernel, h by FC1's epilogue).
#include "common.h"
#include "kernels.h"

namespace bitmoe {

// ------------------------------------------------------------------ 2-bit decoding
// Group table: lut bytes = high bytes of bf16(-4s), bf16(-s), bf16(s), bf16(4s); lb = low byte.
__device__ __forceinline__ void w2_table(uint32_t s16, uint32_t& lut, uint32_t& lb) {
  const uint32_t hb = (s16 >> 8) & 0xFFu;
  lut = ((hb * 0x01010101u) ^ 0x00008080u) + 0x01000001u;
  lb = s16 & 0xFFu;
}

// One MFMA operand (four bf16 pairs) from a code word.  HALF 0 covers s = 0, 1 and HALF 1
// s = 2, 3; for each s: dword (code s, code 4+s), dword (code 8+s, code 12+s).
template <int HALF>
__device__ __forceinline__ u32x4 w2_decode(uint32_t w, uint32_t lut, uint32_t lb) {
  u32x4 r;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sh = 2 * (2 * HALF + u);
    const uint32_t hb = byte_perm(0u, lut, (w >> sh) & 0x03030303u);
    r[2 * u] = byte_perm(lb, hb, 0x01040004u);
    r[2 * u + 1] = byte_perm(lb, hb, 0x03040204u);
  }
  return r;
}

// Slot of k = f (0..15) within 16 consecutive k: the transpose 4*(f%4) + f/4.  For the MFMA
// output row f = 4q + i this is 4i + q.
__device__ __forceinline__ int kpos16(int f) { return 4 * (f & 3) + (f >> 2); }

// ------------------------------------------------------------------ work list
size_t plan_bytes(int64_t max_items) { return (size_t)(16 + 16 * max_items); }

// Block 0 builds the work list; blocks 1.. store x in the k-slot order of the MFMA operand.
//   work list: plan[0] = number of items, then int4 items {expert, first row, rows, hot slot}:
//   the grouped rows of every expert (low-bit experts, or hot experts if want_hot), split
//   into items of at most `chunk` rows, experts in id order.
//   xp[t][16c + p] = x[t][16c + 4*(p%4) + p/4] (the slot order of the MFMA operands).
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
    constexpr uint32_t LO = 0x05040100u, HI = 0x07060302u;
    uint4 o0, o1;
    o0.x = byte_perm(a.z, a.x, LO);  // (x0, x4)
    o0.y = byte_perm(b.z, b.x, LO);  // (x8, x12)
    o0.z = byte_perm(a.z, a.x, HI);  // (x1, x5)
    o0.w = byte_perm(b.z, b.x, HI);  // (x9, x13)
    o1.x = byte_perm(a.w, a.y, LO);  // (x2, x6)
    o1.y = byte_perm(b.w, b.y, LO);  // (x10, x14)
    o1.z = byte_perm(a.w, a.y, HI);  // (x3, x7)
    o1.w = byte_perm(b.w, b.y, HI);  // (x11, x15)
    xp[2 * c] = o0;
    xp[2 * c + 1] = o1;
    return;
  }
  // block 0: the work list
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

constexpr int kRT = 4;  // 16-row A tiles per wave (64 weight rows)

// Lane -> k mapping.  A wave walks its K range in super-steps of G 256-wide steps.  In
// super-step c of step s (0 <= s < G), the lanes of quad q handle the 64 consecutive k
//     kbase + 256*G*c + 64*G*q + 64*s + [0, 64)
// so over a super-step a lane covers 64*G consecutive k: its scales for the whole super-step
// are 4*G contiguous bytes (one load), and its codes for step s are 16 contiguous bytes.
// The token operand uses the same mapping (with the 4x4 slot transpose inside 16 k).

template <int G>
struct ScaleVec;  // a lane's 4*G scale bytes of one super-step: 2*G bf16, two per step
template <> struct ScaleVec<1> { uint32_t v; };
template <> struct ScaleVec<2> { uint32_t v[2]; };
template <> struct ScaleVec<4> { u32x4 v; };

template <int G>
__device__ __forceinline__ ScaleVec<G> load_scales(buf_rsrc r, uint32_t off) {
  ScaleVec<G> sv;
  if constexpr (G == 1) {
    sv.v = buf_load4(r, off);
  } else if constexpr (G == 2) {
    const uint64_t t = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
    sv.v[0] = (uint32_t)t;
    sv.v[1] = (uint32_t)(t >> 32);
  } else {
    sv.v = buf_load16(r, off);
  }
  return sv;
}

template <int G>
__device__ __forceinline__ uint32_t scale_word(const ScaleVec<G>& sv, int s) {
  if constexpr (G == 1) return sv.v;
  else return sv.v[s];
}

// Per-wave pipeline state: code words of steps in a two-slot ring (issued two steps ahead),
// the scales of the current and the next super-step, the token operand in double-buffered
// batches of WB code words, and the accumulators.
template <int NT, int G>
struct W2Pipe {
  static constexpr int WB = NT == 1 ? 4 : 2;  // code words per token batch
  static constexpr int NBATCH = 4 / WB;       // batches per step
  u32x4 cw[2][kRT];
  ScaleVec<G> sc[kRT], sc_next[kRT];
  u32x4 b[2][WB][NT][2];
  f32x4 acc[kRT][NT];
};

// Loads of step `st` (wave-relative) into ring slot `slot`.
template <int NT, int G>
__device__ __forceinline__ void w2_load_codes(W2Pipe<NT, G>& P, int slot, buf_rsrc rc,
                                              const uint32_t* coff, int st) {
  const uint32_t o = 64u * G * (uint32_t)(st / G) + 16u * (uint32_t)(st % G);
#pragma unroll
  for (int t = 0; t < kRT; ++t) P.cw[slot][t] = buf_load16(rc, coff[t] + o);
}

template <int NT, int G>
__device__ __forceinline__ void w2_load_scales(W2Pipe<NT, G>& P, buf_rsrc rs,
                                               const uint32_t* soff, int c) {
#pragma unroll
  for (int t = 0; t < kRT; ++t) P.sc_next[t] = load_scales<G>(rs, soff[t] + 16u * G * (uint32_t)c);
}

// Token operand of batch wb of step `st`.  boff: byte offset of the lane's token row plus its
// quad's k offset, or >= kOffNone for lanes past the item's rows (they read zeros).
template <int NT, int G>
__device__ __forceinline__ void w2_load_batch(W2Pipe<NT, G>& P, int buf, buf_rsrc rb,
                                              const uint32_t* boff, int st, int wb) {
  const uint32_t o = 512u * G * (uint32_t)(st / G) + 128u * (uint32_t)(st % G);
#pragma unroll
  for (int v = 0; v < W2Pipe<NT, G>::WB; ++v) {
    const int j = wb * W2Pipe<NT, G>::WB + v;
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) {
      const uint32_t ob = boff[bt] + o + 32u * j;
      P.b[buf][v][bt][0] = buf_load16(rb, ob);
      P.b[buf][v][bt][1] = buf_load16(rb, ob + 16u);
    }
  }
}

// Step st (wave-relative; ring slot SLOT, position S in its super-step).  Every load is
// unconditional (indices past the range are clamped to the last step, a cache hit), so the
// compiler can count outstanding loads exactly; scheduling barriers keep the prefetches
// where they are issued.
template <int NT, int G, int SLOT, int S>
__device__ __forceinline__ void w2_step(W2Pipe<NT, G>& P, buf_rsrc rc, buf_rsrc rb,
                                        const uint32_t* coff, const uint32_t* boff, int st,
                                        int n_it) {
  constexpr int WB = W2Pipe<NT, G>::WB, NB = W2Pipe<NT, G>::NBATCH;
  uint32_t lut[kRT][2], lb[kRT][2];
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    const uint32_t sw = scale_word<G>(P.sc[t], S);
    w2_table(sw & 0xFFFFu, lut[t][0], lb[t][0]);
    w2_table(sw >> 16, lut[t][1], lb[t][1]);
  }
#pragma unroll
  for (int wb = 0; wb < NB; ++wb) {
    const int buf = NB == 1 ? SLOT : (wb & 1);  // static batch parity
    if (wb + 1 < NB)
      w2_load_batch<NT, G>(P, buf ^ 1, rb, boff, st, wb + 1);
    else
      w2_load_batch<NT, G>(P, buf ^ 1, rb, boff, min(st + 1, n_it - 1), 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < WB; ++v) {
      const int j = wb * WB + v, g = j >> 1;
#pragma unroll
      for (int t = 0; t < kRT; ++t) {
        const u32x4 a = w2_decode<0>(P.cw[SLOT][t][j], lut[t][g], lb[t][g]);
#pragma unroll
        for (int bt = 0; bt < NT; ++bt)
          P.acc[t][bt] = mfma_16x16x32_bf16(a, P.b[buf][v][bt][0], P.acc[t][bt]);
      }
#pragma unroll
      for (int t = 0; t < kRT; ++t) {
        const u32x4 a = w2_decode<1>(P.cw[SLOT][t][j], lut[t][g], lb[t][g]);
#pragma unroll
        for (int bt = 0; bt < NT; ++bt)
          P.acc[t][bt] = mfma_16x16x32_bf16(a, P.b[buf][v][bt][1], P.acc[t][bt]);
      }
    }
  }
  w2_load_codes<NT, G>(P, SLOT, rc, coff, min(st + 2, n_it - 1));
  __builtin_amdgcn_sched_barrier(0);
}

// One super-step (G steps) starting at wave-relative step st0 = G*c; the ring slot of step
// st0 + s is (st0 + s) % 2, which is static because G is even or the caller alternates.
template <int NT, int G, int SLOT0>
__device__ __forceinline__ void w2_superstep(W2Pipe<NT, G>& P, buf_rsrc rc, buf_rsrc rs,
                                             buf_rsrc rb, const uint32_t* coff,
                                             const uint32_t* soff, const uint32_t* boff, int c,
                                             int n_it) {
  const int n_ss = n_it / G;
#pragma unroll
  for (int t = 0; t < kRT; ++t) P.sc[t] = P.sc_next[t];
  w2_load_scales<NT, G>(P, rs, soff, min(c + 1, n_ss - 1));
  __builtin_amdgcn_sched_barrier(0);
  w2_step<NT, G, SLOT0, 0>(P, rc, rb, coff, boff, G * c, n_it);
  if constexpr (G >= 2) w2_step<NT, G, SLOT0 ^ 1, 1>(P, rc, rb, coff, boff, G * c + 1, n_it);
  if constexpr (G == 4) {
    w2_step<NT, G, SLOT0, 2>(P, rc, rb, coff, boff, G * c + 2, n_it);
    w2_step<NT, G, SLOT0 ^ 1, 3>(P, rc, rb, coff, boff, G * c + 3, n_it);
  }
}

// One wave's task: 64 weight rows (4 A tiles) x a K range, for the NT*16 tokens of one item.
//   FC == 1: tiles 0,1 = gate rows 32rb + [0,32), tiles 2,3 = up rows I + 32rb + [0,32) of W1;
//            epilogue h[r][32rb + c] = silu(gate) * up, stored bf16 in k-slot order.
//   FC == 2: tiles t = rows 64rb + 16t + [0,16) of W2; epilogue y[r][64rb + 16t + f] (fp32).
// The 4 waves of a workgroup take 4/KS row blocks x KS parts of K; K parts are summed in LDS.
template <int FC, int NT, int G>
__device__ __forceinline__ void w2_task(const uint32_t* __restrict__ codes,
                                        const uint16_t* __restrict__ scales, size_t ebase,
                                        int rows_per_expert, int K, int width, int ktop,
                                        const uint16_t* __restrict__ bsrc, uint32_t bsrc_bytes,
                                        const int32_t* __restrict__ perm, int blk_rb, int KS,
                                        int r0, int nrows, void* __restrict__ out,
                                        f32x4 (*red)[kRT][kWave]) {
  const int lane = wave_lane(), w = threadIdx.x / kWave;
  const int i16 = lane & 15, q = lane >> 4;
  const int kpart = w % KS, rb_i = blk_rb * (4 / KS) + w / KS;
  const int n_it = (K / 256) / KS;      // steps of this wave (a multiple of G)
  const int k0 = 256 * n_it * kpart;    // first k of this wave
  const int wpr = K / 16, spr = K / 32;
  // per-expert buffers (uniform base, byte size) and per-lane byte offsets
  const buf_rsrc rc = make_rsrc(codes + ebase * wpr, (uint32_t)(rows_per_expert * wpr * 4));
  const buf_rsrc rs = make_rsrc(scales + ebase * spr, (uint32_t)(rows_per_expert * spr * 2));
  const buf_rsrc rb = make_rsrc(bsrc, bsrc_bytes);
  uint32_t coff[kRT], soff[kRT];
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    const int row = FC == 1 ? (t < 2 ? 32 * rb_i + 16 * t : width + 32 * rb_i + 16 * (t - 2)) + i16
                            : 64 * rb_i + 16 * t + i16;
    coff[t] = (uint32_t)(row * wpr * 4 + k0 / 4 + 16 * G * q);
    soff[t] = (uint32_t)(row * spr * 2 + k0 / 16 + 4 * G * q);
  }
  uint32_t boff[NT];
#pragma unroll
  for (int bt = 0; bt < NT; ++bt) {
    const int n = 16 * bt + i16;
    boff[bt] = kOffNone;
    if (n < nrows) {
      const uint32_t rowb = FC == 1 ? (uint32_t)(perm[r0 + n] / ktop) : (uint32_t)(r0 + n);
      boff[bt] = (rowb * (uint32_t)K + (uint32_t)k0 + 64u * G * q) * 2u;
    }
  }
  W2Pipe<NT, G> P;
#pragma unroll
  for (int t = 0; t < kRT; ++t)
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) P.acc[t][bt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // prologue: scales of super-step 0, codes of steps 0 and 1, token batch 0
  w2_load_scales<NT, G>(P, rs, soff, 0);
  w2_load_codes<NT, G>(P, 0, rc, coff, 0);
  w2_load_codes<NT, G>(P, 1, rc, coff, min(1, n_it - 1));
  w2_load_batch<NT, G>(P, 0, rb, boff, 0, 0);
  const int n_ss = n_it / G;
  if constexpr (G == 1) {
    int c = 0;
    for (; c + 1 < n_ss; c += 2) {
      w2_superstep<NT, G, 0>(P, rc, rs, rb, coff, soff, boff, c, n_it);
      w2_superstep<NT, G, 1>(P, rc, rs, rb, coff, soff, boff, c + 1, n_it);
    }
    if (c < n_ss) w2_superstep<NT, G, 0>(P, rc, rs, rb, coff, soff, boff, c, n_it);
  } else {
    for (int c = 0; c < n_ss; ++c) w2_superstep<NT, G, 0>(P, rc, rs, rb, coff, soff, boff, c, n_it);
  }

  // Epilogue, one token tile at a time.  With KS > 1 the K parts of the waves that share a
  // row block are summed through LDS in a fixed order.
#pragma unroll
  for (int bt = 0; bt < NT; ++bt) {
    f32x4 v[kRT];
    if (KS > 1) {
#pragma unroll
      for (int t = 0; t < kRT; ++t) red[w][t][lane] = P.acc[t][bt];
      __syncthreads();
      const int w0 = w - kpart;  // first wave of this row block
#pragma unroll
      for (int t = 0; t < kRT; ++t) {
        f32x4 a = red[w0][t][lane];
        for (int p = 1; p < KS; ++p) a += red[w0 + p][t][lane];
        v[t] = a;
      }
    } else {
#pragma unroll
      for (int t = 0; t < kRT; ++t) v[t] = P.acc[t][bt];
    }
    const int n = 16 * bt + i16;
    if (kpart == 0 && n < nrows) {
      const size_t r = (size_t)(r0 + n);
      if (FC == 1) {
        uint16_t* h = reinterpret_cast<uint16_t*>(out) + r * width + 32 * rb_i;
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gt = v[p][i], up = v[2 + p][i];
            const float hv = __fdividef(gt, 1.0f + __expf(-gt)) * up;
            h[16 * p + kpos16(4 * q + i)] = (uint16_t)f32_to_bf16_rne(hv);
          }
      } else {
        float* y = reinterpret_cast<float*>(out) + r * width + 64 * rb_i + 4 * q;
#pragma unroll
        for (int t = 0; t < kRT; ++t) *reinterpret_cast<f32x4*>(y + 16 * t) = v[t];
      }
    }
    if (KS > 1) __syncthreads();
  }
}

// Tasks (item, row-block group) in a grid-stride loop; an item (<= 32 rows) uses one or two
// 16-token tiles.
template <int FC, int G>
__global__ __launch_bounds__(256, 2) void w2_stream_kernel(
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales, int rows_per_expert,
    int K, int width, int ktop, const uint16_t* __restrict__ bsrc, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ plan, uint32_t bsrc_bytes, int KS, void* __restrict__ out) {
  __shared__ f32x4 red[4][kRT][kWave];
  const int n_items = plan[0];
  const int4* items = reinterpret_cast<const int4*>(plan + 4);
  const int rb_per_item = FC == 1 ? width / 32 : rows_per_expert / 64;
  const int ngrp = rb_per_item / (4 / KS);
  const int total = n_items * ngrp;
  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    const int item = task / ngrp, grp = task - item * ngrp;
    const int4 itm = items[item];
    const size_t ebase = (size_t)itm.x * rows_per_expert;
    const int r0 = itm.y, nrows = itm.z;
    if (nrows <= 16)
      w2_task<FC, 1, G>(codes, scales, ebase, rows_per_expert, K, width, ktop, bsrc, bsrc_bytes, perm,
                        grp, KS, r0, nrows, out, red);
    else
      w2_task<FC, 2, G>(codes, scales, ebase, rows_per_expert, K, width, ktop, bsrc, bsrc_bytes, perm,
                        grp, KS, r0, nrows, out, red);
  }
}

static int grid_for(int64_t tasks) {
  const int64_t cap = 256 * 2;  // resident workgroups (2 per CU): no idle tail blocks
  return (int)(tasks < cap ? (tasks > 0 ? tasks : 1) : cap);
}

// K split across the waves of a workgroup, from the batch size: few tokens -> few busy
// experts -> split K to keep every CU streaming; many tokens -> long K ranges per wave.
// Each part keeps at least 4 steps.
static int k_split_for(int T, int K) {
  int ks = T <= 2 ? 4 : (T <= 16 ? 2 : 1);
  while (ks > 1 && ((K / 256) % ks != 0 || (K / 256) / ks < 4)) ks /= 2;
  return ks;
}

// Super-step length: the largest of 4, 2, 1 dividing the steps of a wave.
static int super_step_for(int K, int ks) {
  const int n = (K / 256) / ks;
  return n % 4 == 0 ? 4 : (n % 2 == 0 ? 2 : 1);
}

template <int FC>
static hipError_t launch_w2(const uint32_t* codes, const uint16_t* scales, int rows, int K,
                            int width, int ktop, const uint16_t* bsrc, const int32_t* perm,
                            const int32_t* plan, uint32_t bsrc_bytes, int ks, int64_t tasks,
                            hipStream_t s, void* out) {
  const int g = super_step_for(K, ks), grid = grid_for(tasks);
  if (g == 4)
    w2_stream_kernel<FC, 4><<<grid, 256, 0, s>>>(codes, scales, rows, K, width, ktop, bsrc, perm, plan, bsrc_bytes, ks, out);
  else if (g == 2)
    w2_stream_kernel<FC, 2><<<grid, 256, 0, s>>>(codes, scales, rows, K, width, ktop, bsrc, perm, plan, bsrc_bytes, ks, out);
  else
    w2_stream_kernel<FC, 1><<<grid, 256, 0, s>>>(codes, scales, rows, K, width, ktop, bsrc, perm, plan, bsrc_bytes, ks, out);
  return hipGetLastError();
}

hipError_t launch_lowbit_fc1(const LowbitWeights& w, int E, int H, int I, int k,
                             const uint16_t* xp, const int32_t* perm, const int32_t* plan,
                             int max_items, int T, uint16_t* hbuf, hipStream_t s) {
  (void)E;
  if (w.fmt != 1) return hipErrorInvalidValue;
  const int ks = k_split_for(T, H);
  const int64_t tasks = (int64_t)max_items * ((I / 32) / (4 / ks));
  return launch_w2<1>((const uint32_t*)w.w1_codes, (const uint16_t*)w.w1_scales, 2 * I, H, I, k,
                      xp, perm, plan, (uint32_t)((size_t)T * H * 2), ks, tasks, s, hbuf);
}

hipError_t launch_lowbit_fc2(const LowbitWeights& w, int E, int H, int I, int k,
                             const uint16_t* hbuf, const int32_t* plan, int max_items, int T,
                             float* y, hipStream_t s) {
  (void)E;
  if (w.fmt != 1) return hipErrorInvalidValue;
  const int ks = k_split_for(T, I);
  const int64_t tasks = (int64_t)max_items * ((H / 64) / (4 / ks));
  return launch_w2<2>((const uint32_t*)w.w2_codes, (const uint16_t*)w.w2_scales, H, I, H, 1, hbuf,
                      nullptr, plan, (uint32_t)((size_t)T * k * I * 2), ks, tasks, s, y);
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
  uint32_t lut, lb;
  w2_table(s16, lut, lb);
  const uint32_t wd = codes[i];
  const u32x4 p0 = w2_decode<0>(wd, lut, lb), p1 = w2_decode<1>(wd, lut, lb);
  float* o = out + row * K + 16 * wc;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    // operand HALF h, pair u: s = 2h + u; dwords (s, 4+s) and (8+s, 12+s)
    o[u] = bf16_to_f32(p0[2 * u] & 0xFFFFu);
    o[4 + u] = bf16_to_f32(p0[2 * u] >> 16);
    o[8 + u] = bf16_to_f32(p0[2 * u + 1] & 0xFFFFu);
    o[12 + u] = bf16_to_f32(p0[2 * u + 1] >> 16);
    o[2 + u] = bf16_to_f32(p1[2 * u] & 0xFFFFu);
    o[6 + u] = bf16_to_f32(p1[2 * u] >> 16);
    o[10 + u] = bf16_to_f32(p1[2 * u + 1] & 0xFFFFu);
    o[14 + u] = bf16_to_f32(p1[2 * u + 1] >> 16);
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
