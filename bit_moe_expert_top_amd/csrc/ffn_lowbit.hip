// Expert FFN over low-bit codebook weights: weight-streaming kernels with MFMA on 16-token
// tiles (the decode shape: few tokens per expert, every weight byte read once).
//
// [Moet-QA] (2-bit experts on the codebook {-4,-1,1,4}, a bf16 scale per 32 along K);
// [Strata-R9700] path 6 (3-bit experts, eight levels, an e4m3 scale / 64 per 64 along K);
// [Moet-README] release notes of -r23: each expert is FC1 (gate and up), SwiGLU, then FC2.
//
// Work split.  A task is (chunk of <= 16*NT grouped rows of one expert, 64*4/KS weight rows);
// a workgroup of 4 waves takes a task, each wave 64 rows and one of KS parts of K.  Each wave
// streams its rows' packed codes (16 or 24 bytes per lane per 64 k), decodes them to exact bf16
// in registers (lowbit_fmt.h) and feeds v_mfma_f32_16x16x32_bf16 with the weights as A
// (16 rows x 32 k) and the tokens as B (32 k x 16 tokens).  The K parts are summed in LDS in a
// fixed order (deterministic), then FC1 applies SwiGLU and stores h (bf16), FC2 stores y (fp32).
// The token operand is stored in the format's k-slot order (x by the prepare kernel, h by
// FC1's epilogue), so A and B agree slot by slot.
#include "common.h"
#include "kernels.h"
#include "lowbit_fmt.h"
#include "plan.h"

namespace bitmoe {

// ------------------------------------------------------------------ work list
size_t plan_bytes(int64_t max_items) { return (size_t)(16 + 16 * max_items); }

// Block 0 builds the work lists; blocks 1.. store x in the k-slot order of the weight format.
//   work lists (build_plan2): the grouped rows of every low-bit expert, in items of at most
//   `small_max` rows for the streaming kernel, or (gemm_enabled, groups above small_max) of at
//   most `gemm_chunk` rows for the grouped GEMM; experts in id order.
//   x in slot order: x_chunk_to_slots (one thread per 16 k for 2-bit, per 32 k for 3-bit).
__global__ __launch_bounds__(1024) void prepare_kernel(const int32_t* __restrict__ offsets, int E,
                                                       int small_max, int gemm_chunk, int gemm_enabled,
                                                       const int32_t* __restrict__ hot_ids, int n_hot,
                                                       int hot_residual, int32_t* __restrict__ plan_s,
                                                       int32_t* __restrict__ plan_g,
                                                       const uint4* __restrict__ x, int nchunks,
                                                       int fmt, uint4* __restrict__ xp) {
  if (blockIdx.x > 0) {
    const int c = (blockIdx.x - 1) * 1024 + threadIdx.x;
    if (c >= nchunks) return;
    x_chunk_to_slots(x, c, fmt, xp);
    return;
  }
  build_plan2(offsets, E, small_max, gemm_chunk, gemm_enabled, hot_ids, n_hot, hot_residual, plan_s, plan_g);
}

hipError_t launch_prepare(const int32_t* offsets, int E, int small_max, int gemm_chunk, bool gemm_enabled,
                          const int32_t* hot_ids, int n_hot, bool hot_residual, int32_t* plan_s,
                          int32_t* plan_g, const uint16_t* x, int T, int H, int fmt, uint16_t* xp,
                          hipStream_t s) {
  const int per = fmt == W2Fmt::kId ? 16 : 32;  // k per thread
  const int nchunks = xp ? T * (H / per) : 0;
  const int blocks = 1 + (nchunks + 1023) / 1024;
  prepare_kernel<<<blocks, 1024, 0, s>>>(offsets, E, small_max, gemm_chunk, gemm_enabled ? 1 : 0, hot_ids,
                                         n_hot, hot_residual ? 1 : 0, plan_s, plan_g, (const uint4*)x, nchunks,
                                         fmt, (uint4*)xp);
  return hipGetLastError();
}

// ------------------------------------------------------------------ the streaming kernel

constexpr int kRT = 4;  // 16-row A tiles per wave (64 weight rows)

// Lane -> k mapping.  A wave walks its K range in super-steps of G (1 or 2) 64-k steps per
// quad.  In super-step c, step s (0 <= s < G), the lanes of quad q handle the 64 consecutive k
//     kbase + 256*G*c + 64*G*q + 64*s + [0, 64)
// so over a super-step a lane covers 64*G consecutive k and the four quads of a row 256*G
// consecutive k: with G = 2 and 2-bit codes that is one whole 128-byte line per row, requested
// by one group of loads issued together (lines split over loads issued far apart were evicted
// from the L2 between their uses and fetched again).  A lane's scales for the super-step are
// contiguous bytes (one load).
//
// The token operand (B) of a step is staged in LDS once per workgroup and shared by its 4
// waves: direct global -> LDS loads (16 bytes per lane, no registers), double buffered, one
// barrier per step.  A stage holds, for each of the KS parts of K, the 16*NT token rows of the
// item, each 256 k (512 bytes, the step's four 64-k pieces in quad order) with the 16-byte
// chunks XOR-swizzled by the token index (conflict-free LDS reads).
constexpr int kBStage = 4 * 16 * 512;  // the largest stage: KS = 4 x 16 tokens (or KS = 1 x 32)
typedef __attribute__((address_space(3))) void lds_void;

// Per-wave pipeline state of one pass over K: the weight resources and this lane's offsets, the
// codes of two super-steps (the current one and the next, issued one super-step ahead), the
// scales of the current and the next super-step.  The accumulators live outside, so that a
// second pass (the FP4 residual of a hot expert) adds into the same sums.
template <class F, int NT, int G>
struct Pipe {
  static constexpr int SB = F::kStepScaleBytes * G;
  buf_rsrc rc, rs;
  uint32_t coff[kRT], soff[kRT];
  typename F::Codes cw[2][G][kRT];
  ScaleBytes<SB> sc[kRT], sc_next[kRT];
};

// Codes of super-step c (all G steps, issued together) into ring slot `slot`.
template <class F, int NT, int G>
__device__ __forceinline__ void load_codes(Pipe<F, NT, G>& P, int slot, int c) {
#pragma unroll
  for (int t = 0; t < kRT; ++t)
#pragma unroll
    for (int s = 0; s < G; ++s)
      P.cw[slot][s][t] = F::load_codes_s(P.rc, P.coff[t], F::code_bytes(256u * G * (uint32_t)c + 64u * (uint32_t)s));
}

template <class F, int NT, int G>
__device__ __forceinline__ void load_scales(Pipe<F, NT, G>& P, int c) {
#pragma unroll
  for (int t = 0; t < kRT; ++t)
    P.sc_next[t] = load_scale_bytes_s<Pipe<F, NT, G>::SB>(P.rs, P.soff[t], F::scale_bytes(256u * G * (uint32_t)c));
}

// The weight resources of one expert (or one hot slot of the residual arrays) and this lane's
// code and scale offsets: tile t of the wave is weight row row[t] + (lane % 16); the lane's
// k range starts at kq.
template <class F, int NT, int G>
__device__ __forceinline__ void pipe_init(Pipe<F, NT, G>& P, const uint8_t* __restrict__ codes,
                                          const uint8_t* __restrict__ scales, size_t ebase, int rows_per_expert,
                                          int K, const int* row, int kq) {
  const uint32_t cbr = F::code_bytes((uint32_t)K), sbr = F::scale_bytes((uint32_t)K);
  P.rc = make_rsrc(codes + ebase * cbr, (uint32_t)rows_per_expert * cbr);
  P.rs = make_rsrc(scales + ebase * sbr, (uint32_t)rows_per_expert * sbr);
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    P.coff[t] = (uint32_t)row[t] * cbr + F::code_bytes((uint32_t)kq);
    P.soff[t] = (uint32_t)row[t] * sbr + F::scale_bytes((uint32_t)kq);
  }
}

// Direct loads of the token operand of step st into a stage buffer: round u of this wave
// writes the 1 KB at stage + 16 * (256 u + 64 w).  doff: per-round source offsets (>= kOffNone
// for chunks past the item's rows, which land as zeros).
// `active` (wave-uniform) has bit u set for the rounds of this wave that hold a real token.
template <int G>
__device__ __forceinline__ void dma_b(buf_rsrc rb, uint8_t* stage, const uint32_t* doff, uint32_t active,
                                      int wu, int st) {
  const uint32_t ko = 2u * (256u * G * (uint32_t)(st / G) + 64u * (uint32_t)(st % G));
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (active & (1u << u))
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(stage + 16 * (256 * u + 64 * wu)), 16,
                                               (int)doff[u], (int)ko, 0, 0);
}

// s_waitcnt vmcnt(N) on gfx9: vmcnt in bits [3:0] and [15:14]; expcnt (bits [6:4]) and lgkmcnt
// (bits [11:8]) at their maximum, i.e. not waited on.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}

// Step st = G*c + S of super-step c (code ring slot CS, B stage BS = st % 2).
//   1. wait for this wave's loads of B(st) -- vector loads complete in issue order, so at S = 1
//      the next super-step's codes and scales (issued after B(st)) may stay in flight -- then
//      a barrier: B(st) of every wave is in LDS and every wave is done with B(st-1);
//   2. issue B(st+1) into the other stage; at S = 0 then issue the codes and scales of
//      super-step c+1 (not in the last super-step, LAST, whose S = 1 step then waits for
//      everything); decode + MFMA, the token operands read one operand ahead of their MFMAs
//      (the LDS latency hides behind the decode).
template <class F, int NT, int G, int CS, int BS, int S, bool LAST>
__device__ __forceinline__ void step(Pipe<F, NT, G>& P, f32x4 (&acc)[kRT][NT], buf_rsrc rb, uint8_t* bs0,
                                     uint8_t* bs1, const uint32_t* doff, uint32_t active, int wu,
                                     const uint32_t* bread, int c, int n_it) {
  constexpr int kLc = F::kStepCodeBytes > 16 ? 2 : 1;  // load instructions per tile and step
  constexpr int kAfter = S == 1 && !LAST ? kRT * (1 + G * kLc) : 0;
  const int st = G * c + S;
  wait_vmcnt<kAfter>();
  __syncthreads();
  if (st + 1 < n_it) dma_b<G>(rb, BS ? bs0 : bs1, doff, active, wu, st + 1);
  if constexpr (S == 0) {
#pragma unroll
    for (int t = 0; t < kRT; ++t) P.sc[t] = P.sc_next[t];
    if constexpr (!LAST) {
      load_scales<F, NT, G>(P, c + 1);
      load_codes<F, NT, G>(P, CS ^ 1, c + 1);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint8_t* bsrc = BS ? bs1 : bs0;
  typename F::Tab tab[kRT];
#pragma unroll
  for (int t = 0; t < kRT; ++t) tab[t] = F::table(F::step_scale(P.sc[t], S));
  u32x4 b[2][NT];
#pragma unroll
  for (int bt = 0; bt < NT; ++bt) b[0][bt] = *reinterpret_cast<const u32x4*>(bsrc + bread[bt * 8]);
#pragma unroll
  for (int o = 0; o < 8; ++o) {
    if (o + 1 < 8) {
#pragma unroll
      for (int bt = 0; bt < NT; ++bt)
        b[(o + 1) & 1][bt] = *reinterpret_cast<const u32x4*>(bsrc + bread[bt * 8 + o + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the next operand's reads ahead of this decode
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
      const u32x4 a = F::decode(P.cw[CS][S][t], tab[t], o);
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) acc[t][bt] = mfma_16x16x32_bf16(a, b[o & 1][bt], acc[t][bt]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// One super-step c (code ring slot CS = c % 2).
template <class F, int NT, int G, int CS, bool LAST>
__device__ __forceinline__ void superstep(Pipe<F, NT, G>& P, f32x4 (&acc)[kRT][NT], buf_rsrc rb, uint8_t* bs0,
                                          uint8_t* bs1, const uint32_t* doff, uint32_t active, int wu,
                                          const uint32_t* bread, int c, int n_it) {
  // B stage of step G*c + S is its parity: S for G = 2, CS for G = 1
  step<F, NT, G, CS, (G == 1 ? CS : 0), 0, LAST>(P, acc, rb, bs0, bs1, doff, active, wu, bread, c, n_it);
  if constexpr (G == 2) step<F, NT, G, CS, 1, 1, LAST>(P, acc, rb, bs0, bs1, doff, active, wu, bread, c, n_it);
}

// The super-steps of one pass (the prologue's loads of super-step 0 and of B(0) issued).  The
// last one is peeled off the loop: it loads no next super-step.
template <class F, int NT, int G>
__device__ __forceinline__ void stream_loop(Pipe<F, NT, G>& P, f32x4 (&acc)[kRT][NT], buf_rsrc rb, uint8_t* bs0,
                                            uint8_t* bs1, const uint32_t* doff, uint32_t active, int wu,
                                            const uint32_t* bread, int n_it) {
  const int n_ss = n_it / G;  // >= 1
  int c = 0;
  for (; c + 2 < n_ss; c += 2) {
    superstep<F, NT, G, 0, false>(P, acc, rb, bs0, bs1, doff, active, wu, bread, c, n_it);
    superstep<F, NT, G, 1, false>(P, acc, rb, bs0, bs1, doff, active, wu, bread, c + 1, n_it);
  }
  if (c + 2 == n_ss) {
    superstep<F, NT, G, 0, false>(P, acc, rb, bs0, bs1, doff, active, wu, bread, c, n_it);
    superstep<F, NT, G, 1, true>(P, acc, rb, bs0, bs1, doff, active, wu, bread, c + 1, n_it);
  } else {
    superstep<F, NT, G, 0, true>(P, acc, rb, bs0, bs1, doff, active, wu, bread, c, n_it);
  }
}

// Source offsets of this lane's direct B loads (one per 256-chunk round u of the workgroup) for
// super-steps of G steps: chunk c of token n of K part p (position c ^ (n & 7) in the token's
// 512 bytes of the stage) holds the 8 k at 64*G*(c/8) + 8*(c%8) of the part's current step.
// Rounds past the item's rows get kOffNone (they load zeros).
template <int NT, int G>
__device__ __forceinline__ void b_offsets(uint32_t* doff, int w, int lane, int nrows, int K, int n_it, int nrounds,
                                          uint32_t lane_row) {
  const int per_part = NT * 16 * 32;  // chunks per K part
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int f = 256 * u + 64 * w + lane;
    const int p = f / per_part, rem = f - p * per_part, n = rem >> 5, pos = rem & 31;
    const int c = pos ^ (n & 7);
    const int nn = min(n, nrows - 1);
    const uint32_t rowb = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * nn, (int)lane_row);
    const uint32_t o = (rowb * (uint32_t)K + (uint32_t)(256 * n_it * p) + 64u * G * (uint32_t)(c >> 3)) * 2u +
                       16u * (uint32_t)(c & 7);
    doff[u] = (u < nrounds && n < nrows) ? o : kOffNone;
  }
}

// One wave's task: 64 weight rows (4 A tiles) x a K range, for the NT*16 tokens of one item.
//   FC == 1: tiles 0,1 = gate rows 32rb + [0,32), tiles 2,3 = up rows I + 32rb + [0,32) of W1;
//            epilogue h[r][32rb + pos32(c)] = silu(gate) * up for c in [0,32), stored bf16.
//   FC == 2: tiles t = rows 64rb + 16t + [0,16) of W2; epilogue y[r][64rb + 16t + f] (fp32).
// The 4 waves of a workgroup take 4/KS row blocks x KS parts of K; K parts are summed in LDS.
// RES: a hot expert of a layer with an FP4 residual (rslot >= 0) makes a second pass over the
// same rows and k with the residual's MXFP4 codes, into the same accumulators.
template <class F, int FC, int NT, int G, bool RES>
__device__ __forceinline__ void stream_task(const uint8_t* __restrict__ codes,
                                            const uint8_t* __restrict__ scales, size_t ebase,
                                            int rows_per_expert, int K, int width, int ktop,
                                            const uint16_t* __restrict__ bsrc, uint32_t bsrc_bytes,
                                            const int32_t* __restrict__ perm, int blk_rb, int KS,
                                            int r0, int nrows, void* __restrict__ out, uint8_t* bs0,
                                            uint8_t* bs1, const uint8_t* __restrict__ rcodes,
                                            const uint8_t* __restrict__ rscales, int rslot) {
  const int lane = wave_lane(), w = threadIdx.x / kWave;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int i16 = lane & 15, q = lane >> 4;
  const int kpart = w % KS, rb_i = blk_rb * (4 / KS) + w / KS;
  const int n_it = (K / 256) / KS;      // steps of this wave (a multiple of G)
  const int k0 = 256 * n_it * kpart;    // first k of this wave
  // FC1 gathers token rows of x (all of x is addressable, < 4 GiB); FC2 reads the item's own h
  // rows, so its resource is based at row r0 (h may exceed 4 GiB)
  const buf_rsrc rb = FC == 1 ? make_rsrc(bsrc, bsrc_bytes)
                              : make_rsrc(bsrc + (size_t)r0 * K, (uint32_t)nrows * (uint32_t)K * 2u);
  // Source row of each of the item's (<= 32) tokens: lane i looks up token i once (one
  // branch-free load, issued before the prologue's code loads so the two latencies overlap),
  // and the B rounds below read it from that lane.
  uint32_t lane_row = (uint32_t)min(lane & 31, nrows - 1);
  uint32_t perm_v = 0;
  if constexpr (FC == 1) perm_v = (uint32_t)perm[r0 + (int)lane_row];
  int row[kRT];
#pragma unroll
  for (int t = 0; t < kRT; ++t)
    row[t] = FC == 1 ? (t < 2 ? 32 * rb_i + 16 * t : width + 32 * rb_i + 16 * (t - 2)) + i16
                     : 64 * rb_i + 16 * t + i16;
  const int kq = k0 + 64 * G * q;
  Pipe<F, NT, G> P;
  pipe_init<F, NT, G>(P, codes, scales, ebase, rows_per_expert, K, row, kq);
  f32x4 acc[kRT][NT];
#pragma unroll
  for (int t = 0; t < kRT; ++t)
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) acc[t][bt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // prologue: scales and codes of super-step 0 (B of step 0 below, once its rows are known)
  load_scales<F, NT, G>(P, 0);
  load_codes<F, NT, G>(P, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (FC == 1) lane_row = perm_v / (uint32_t)ktop;
  // B stage: KS parts x 16*NT tokens x 32 chunks of 16 bytes; chunk c of token n sits at
  // position c ^ (n & 7) of the token's 512 bytes.
  const int per_part = NT * 16 * 32;    // chunks per K part
  const int nrounds = KS * NT * 2;      // 256-chunk rounds of the workgroup (<= 8)
  uint32_t doff[8];
  b_offsets<NT, G>(doff, w, lane, nrows, K, n_it, nrounds, lane_row);
  // rounds of this wave that carry at least one real token row (a round of a wave covers the
  // 2 token rows of its 64 chunks); the others are not issued
  uint32_t active = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int n_lo = ((256 * u + 64 * wu) % per_part) >> 5;
    if (u < nrounds && n_lo < nrows) active |= 1u << u;
  }
  uint32_t bread[NT * 8];  // LDS byte offsets of this lane's B operands in a stage
#pragma unroll
  for (int bt = 0; bt < NT; ++bt)
#pragma unroll
    for (int o = 0; o < 8; ++o)
      bread[bt * 8 + o] = (uint32_t)(kpart * per_part * 16 + (16 * bt + i16) * 512 + 16 * ((8 * q + o) ^ (i16 & 7)));

  dma_b<G>(rb, bs0, doff, active, wu, 0);
  __builtin_amdgcn_sched_barrier(0);
  stream_loop<F, NT, G>(P, acc, rb, bs0, bs1, doff, active, wu, bread, n_it);
  if constexpr (RES) {
    if (rslot >= 0) {  // uniform over the workgroup (one item)
      // the residual pass: 32 code bytes per lane and step, so super-steps of one step (a
      // two-step code ring would not fit the registers), with the B offsets of that k mapping
      constexpr int GR = 1;
      __syncthreads();  // every wave is done reading the B stages of the first pass
      Pipe<Fp4Fmt, NT, GR> R;
      pipe_init<Fp4Fmt, NT, GR>(R, rcodes, rscales, (size_t)rslot * rows_per_expert, rows_per_expert, K, row,
                                k0 + 64 * GR * q);
      load_scales<Fp4Fmt, NT, GR>(R, 0);
      load_codes<Fp4Fmt, NT, GR>(R, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      b_offsets<NT, GR>(doff, w, lane, nrows, K, n_it, nrounds, lane_row);
      dma_b<GR>(rb, bs0, doff, active, wu, 0);
      __builtin_amdgcn_sched_barrier(0);
      stream_loop<Fp4Fmt, NT, GR>(R, acc, rb, bs0, bs1, doff, active, wu, bread, n_it);
    }
  }

  // Epilogue, one token tile at a time.  With KS > 1 the K parts of the waves that share a
  // row block are summed through LDS (over the first B stage, free now) in a fixed order.
  f32x4 (*red)[kRT][kWave] = reinterpret_cast<f32x4 (*)[kRT][kWave]>(bs0);
  __syncthreads();  // every wave is done reading the B stages
#pragma unroll
  for (int bt = 0; bt < NT; ++bt) {
    f32x4 v[kRT];
    if (KS > 1) {
#pragma unroll
      for (int t = 0; t < kRT; ++t) red[w][t][lane] = acc[t][bt];
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
      for (int t = 0; t < kRT; ++t) v[t] = acc[t][bt];
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
            h[F::pos32(16 * p + 4 * q + i)] = (uint16_t)f32_to_bf16_rne(hv);
          }
      } else {
        float* y = reinterpret_cast<float*>(out) + r * width + 64 * rb_i + 4 * q;
#pragma unroll
        for (int t = 0; t < kRT; ++t) *reinterpret_cast<f32x4*>(y + 16 * t) = v[t];
      }
    }
    __syncthreads();  // the LDS of this tile / stage is reused by the next tile or task
  }
}

// Tasks (item, row-block group) in a grid-stride loop; an item (<= 32 rows) uses one or two
// 16-token tiles.  With RES, an item whose hot slot (item.w) is >= 0 adds the FP4 residual.
template <class F, int FC, int G, bool RES>
__global__ __launch_bounds__(256, 2) void stream_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int rows_per_expert,
    int K, int width, int ktop, const uint16_t* __restrict__ bsrc, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ plan, uint32_t bsrc_bytes, int KS, void* __restrict__ out,
    const uint8_t* __restrict__ rcodes, const uint8_t* __restrict__ rscales) {
  __shared__ __align__(16) uint8_t bs0[kBStage];
  __shared__ __align__(16) uint8_t bs1[kBStage];
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
    const int rslot = RES ? itm.w : -1;
    if (nrows <= 16)
      stream_task<F, FC, 1, G, RES>(codes, scales, ebase, rows_per_expert, K, width, ktop, bsrc, bsrc_bytes,
                                    perm, grp, KS, r0, nrows, out, bs0, bs1, rcodes, rscales, rslot);
    else
      stream_task<F, FC, 2, G, RES>(codes, scales, ebase, rows_per_expert, K, width, ktop, bsrc, bsrc_bytes,
                                    perm, grp, KS, r0, nrows, out, bs0, bs1, rcodes, rscales, rslot);
  }
}

static int grid_for(int64_t tasks) {
  const int64_t cap = 256 * 2;  // resident workgroups (2 per CU): no idle tail blocks
  return (int)(tasks < cap ? (tasks > 0 ? tasks : 1) : cap);
}

// K split across the waves of a workgroup, from the batch size: few tokens -> few busy
// experts -> split K to keep every CU streaming; many tokens -> long K ranges per wave.
// 3-bit experts (fewer, shorter rows per byte streamed) keep the two-way split up to 127 tokens,
// where it measured faster; for 2-bit it measured slower above 16 tokens.
// Each part keeps at least 4 steps when it can.
static int k_split_for(int T, int K, int fmt) {
  const int two_way_max = fmt == W3Fmt::kId ? 127 : 16;
  int ks = T <= 2 ? 4 : (T <= two_way_max ? 2 : 1);
  while (ks > 1 && ((K / 256) % ks != 0 || (K / 256) / ks < 4)) ks /= 2;
  return ks;
}

// Super-step length: 2 steps when the steps of a wave are even, else 1.
static int super_step_for(int K, int ks) {
  const int n = (K / 256) / ks;
  return n % 2 == 0 ? 2 : 1;
}

template <class F, int FC, bool RES>
static hipError_t launch_stream(const void* codes, const void* scales, int rows, int K, int width,
                                int ktop, const uint16_t* bsrc, const int32_t* perm,
                                const int32_t* plan, uint32_t bsrc_bytes, int ks, int64_t tasks,
                                hipStream_t s, void* out, const void* rcodes, const void* rscales) {
  const int g = super_step_for(K, ks), grid = grid_for(tasks);
  const uint8_t* c = (const uint8_t*)codes;
  const uint8_t* sc = (const uint8_t*)scales;
  const uint8_t* rc = (const uint8_t*)rcodes;
  const uint8_t* rs = (const uint8_t*)rscales;
  if (g == 2)
    stream_kernel<F, FC, 2, RES><<<grid, 256, 0, s>>>(c, sc, rows, K, width, ktop, bsrc, perm, plan, bsrc_bytes, ks,
                                                      out, rc, rs);
  else
    stream_kernel<F, FC, 1, RES><<<grid, 256, 0, s>>>(c, sc, rows, K, width, ktop, bsrc, perm, plan, bsrc_bytes, ks,
                                                      out, rc, rs);
  return hipGetLastError();
}

hipError_t launch_lowbit_fc1(const LowbitWeights& w, int E, int H, int I, int k,
                             const uint16_t* xp, const int32_t* perm, const int32_t* plan,
                             int max_items, int T, int split_T, uint16_t* hbuf, hipStream_t s) {
  (void)E;
  const int ks = k_split_for(split_T, H, w.fmt);
  const int64_t tasks = (int64_t)max_items * ((I / 32) / (4 / ks));
  const uint32_t xb = (uint32_t)((size_t)T * H * 2);
  if (w.fmt == W2Fmt::kId && w.res_w1_codes)
    return launch_stream<W2Fmt, 1, true>(w.w1_codes, w.w1_scales, 2 * I, H, I, k, xp, perm, plan, xb, ks, tasks, s,
                                         hbuf, w.res_w1_codes, w.res_w1_scales);
  if (w.fmt == W2Fmt::kId)
    return launch_stream<W2Fmt, 1, false>(w.w1_codes, w.w1_scales, 2 * I, H, I, k, xp, perm, plan, xb, ks, tasks, s,
                                          hbuf, nullptr, nullptr);
  if (w.fmt == W3Fmt::kId)
    return launch_stream<W3Fmt, 1, false>(w.w1_codes, w.w1_scales, 2 * I, H, I, k, xp, perm, plan, xb, ks, tasks, s,
                                          hbuf, nullptr, nullptr);
  return hipErrorInvalidValue;
}

hipError_t launch_lowbit_fc2(const LowbitWeights& w, int E, int H, int I, int k,
                             const uint16_t* hbuf, const int32_t* plan, int max_items, int T,
                             int split_T, float* y, hipStream_t s) {
  (void)E;
  (void)T;
  const int ks = k_split_for(split_T, I, w.fmt);
  const int64_t tasks = (int64_t)max_items * ((H / 64) / (4 / ks));
  const uint32_t hb = 0;  // unused: FC2 bases its resource at each item's rows
  if (w.fmt == W2Fmt::kId && w.res_w2_codes)
    return launch_stream<W2Fmt, 2, true>(w.w2_codes, w.w2_scales, H, I, H, 1, hbuf, nullptr, plan, hb, ks, tasks, s,
                                         y, w.res_w2_codes, w.res_w2_scales);
  if (w.fmt == W2Fmt::kId)
    return launch_stream<W2Fmt, 2, false>(w.w2_codes, w.w2_scales, H, I, H, 1, hbuf, nullptr, plan, hb, ks, tasks, s,
                                          y, nullptr, nullptr);
  if (w.fmt == W3Fmt::kId)
    return launch_stream<W3Fmt, 2, false>(w.w2_codes, w.w2_scales, H, I, H, 1, hbuf, nullptr, plan, hb, ks, tasks, s,
                                          y, nullptr, nullptr);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ debug decode
// One thread per (row, 64 k): decode with the kernels' own load/table/decode path and write
// the weights in natural k order.
template <class F>
__global__ __launch_bounds__(256) void debug_dequant_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            int rows, int K, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int spr = K / 64;
  if (i >= (int64_t)rows * spr) return;
  const int row = (int)(i / spr), st = (int)(i - (int64_t)row * spr);
  const uint32_t cbr = F::code_bytes((uint32_t)K), sbr = F::scale_bytes((uint32_t)K);
  const buf_rsrc rc = make_rsrc(codes, (uint32_t)rows * cbr);
  const buf_rsrc rs = make_rsrc(scales, (uint32_t)rows * sbr);
  const typename F::Codes c = F::load_codes(rc, (uint32_t)row * cbr + F::code_bytes(64u * st));
  const ScaleBytes<F::kStepScaleBytes> sb =
      load_scale_bytes<F::kStepScaleBytes>(rs, (uint32_t)row * sbr + F::scale_bytes(64u * st));
  const typename F::Tab tab = F::table(F::step_scale(sb, 0));
  float* o = out + (int64_t)row * K + 64 * st;
#pragma unroll
  for (int op = 0; op < 8; ++op) {
    const u32x4 v = F::decode(c, tab, op);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int slot = 8 * op + 2 * d;  // slots of this dword within the 64 k
      o[32 * (slot >> 5) + F::slot_k(slot & 31)] = bf16_to_f32(v[d] & 0xFFFFu);
      o[32 * (slot >> 5) + F::slot_k((slot + 1) & 31)] = bf16_to_f32(v[d] >> 16);
    }
  }
}

hipError_t launch_debug_dequant(const LowbitWeights& w, int E, int H, int I, int e, int which,
                                float* out, hipStream_t s) {
  (void)E;
  const int rows = which == 1 ? 2 * I : H;
  const int K = which == 1 ? H : I;
  const void* codes = which == 1 ? w.w1_codes : w.w2_codes;
  const void* scales = which == 1 ? w.w1_scales : w.w2_scales;
  const int64_t n = (int64_t)rows * (K / 64);
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (w.fmt == W2Fmt::kId) {
    const size_t cb = (size_t)e * rows * W2Fmt::code_bytes(K), sb = (size_t)e * rows * W2Fmt::scale_bytes(K);
    debug_dequant_kernel<W2Fmt><<<grid, 256, 0, s>>>((const uint8_t*)codes + cb, (const uint8_t*)scales + sb,
                                                     rows, K, out);
  } else if (w.fmt == W3Fmt::kId) {
    const size_t cb = (size_t)e * rows * W3Fmt::code_bytes(K), sb = (size_t)e * rows * W3Fmt::scale_bytes(K);
    debug_dequant_kernel<W3Fmt><<<grid, 256, 0, s>>>((const uint8_t*)codes + cb, (const uint8_t*)scales + sb,
                                                     rows, K, out);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_debug_dequant_residual(const LowbitWeights& w, int H, int I, int slot, int which, float* out,
                                         hipStream_t s) {
  const int rows = which == 1 ? 2 * I : H;
  const int K = which == 1 ? H : I;
  const uint8_t* codes = (const uint8_t*)(which == 1 ? w.res_w1_codes : w.res_w2_codes);
  const uint8_t* scales = (const uint8_t*)(which == 1 ? w.res_w1_scales : w.res_w2_scales);
  if (!codes || !scales) return hipErrorInvalidValue;
  const int64_t n = (int64_t)rows * (K / 64);
  const unsigned grid = (unsigned)((n + 255) / 256);
  const size_t cb = (size_t)slot * rows * Fp4Fmt::code_bytes(K), sb = (size_t)slot * rows * Fp4Fmt::scale_bytes(K);
  debug_dequant_kernel<Fp4Fmt><<<grid, 256, 0, s>>>(codes + cb, scales + sb, rows, K, out);
  return hipGetLastError();
}

}  // namespace bitmoe
