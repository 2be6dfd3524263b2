// Hot experts held in MXFP4, computed in FP8 ([Moet-QA]: the hottest experts are kept at FP4
// precision; [Day0-MXFP4] section 4: MXFP4 expert weights are converted online to FP8 into a
// reused workspace before the matmuls; [Moet-README] release notes of -r23: FC1, SwiGLU and
// MXFP8 quantisation, then FC2).
//
//   mxfp8_quant_kernel   x (bf16) -> MXFP8 (e4m3fn elements + e8m0 scale per 32 along H)
//   mxfp4_convert_kernel an MXFP4 matrix -> e4m3fn bytes of the same values + the e8m0 scales
//                        (lossless); the FFN converts every hot expert with tokens into a
//                        workspace slot
//   fp8_gemm_kernel      grouped GEMM on v_mfma_scale_f32_32x32x64_f8f6f4 (the matrix cores
//                        apply the e8m0 block scales): FC1 fuses SwiGLU and the MXFP8
//                        quantisation of h; FC2 stores y (fp32)
//
// The scaled MFMA takes each lane's 32 bytes as two 16-byte chunks: lane l (row l % 32,
// half h = l / 32) holds k = 32c + 16h + [0,16) in chunk c, and its scale operand is the
// e8m0 scale of the 32-k block h.  (Established on the device: data and scales placed this
// way reproduce the fp64 product of the dequantised operands.)
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "mx_fmt.h"
#include "plan.h"

namespace bitmoe {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ MXFP8 of bf16 rows
// One thread per 32-element block: amax, shared exponent, 32 elements.
__device__ __forceinline__ void mxfp8_block(const uint4* __restrict__ x, int64_t i, uint4* __restrict__ elems,
                                            uint8_t* __restrict__ scales) {
  uint32_t w[16];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint4 v = x[4 * i + u];
    w[4 * u] = v.x;
    w[4 * u + 1] = v.y;
    w[4 * u + 2] = v.z;
    w[4 * u + 3] = v.w;
  }
  uint32_t amax = 0;  // bf16 magnitudes order like unsigned integers
#pragma unroll
  for (int d = 0; d < 16; ++d) amax = max(amax, max(w[d] & 0x7FFFu, (w[d] >> 16) & 0x7FFFu));
  const int shared = mx_shared_exp(amax ? floor_log2_bf16(amax) : 0, amax == 0);
  uint32_t o[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    const uint32_t e0 = bf16_to_e4m3_scaled(w[2 * d] & 0xFFFFu, shared);
    const uint32_t e1 = bf16_to_e4m3_scaled(w[2 * d] >> 16, shared);
    const uint32_t e2 = bf16_to_e4m3_scaled(w[2 * d + 1] & 0xFFFFu, shared);
    const uint32_t e3 = bf16_to_e4m3_scaled(w[2 * d + 1] >> 16, shared);
    o[d] = e0 | (e1 << 8) | (e2 << 16) | (e3 << 24);
  }
  elems[2 * i] = make_uint4(o[0], o[1], o[2], o[3]);
  elems[2 * i + 1] = make_uint4(o[4], o[5], o[6], o[7]);
  scales[i] = (uint8_t)(shared + 127);
}

__global__ __launch_bounds__(256) void mxfp8_quant_kernel(const uint4* __restrict__ x, int64_t nblocks,
                                                          uint4* __restrict__ elems,
                                                          uint8_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nblocks) mxfp8_block(x, i, elems, scales);
}

// Block 0: the hot work list; blocks 1..: MXFP8 of every token row of x (the FC1 input of the
// hot experts).
__global__ __launch_bounds__(1024) void hot_prepare_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int chunk, const int32_t* __restrict__ hot_ids,
                                                           int n_hot, int32_t* __restrict__ plan,
                                                           const uint4* __restrict__ x, int64_t nblocks,
                                                           uint4* __restrict__ elems,
                                                           uint8_t* __restrict__ scales) {
  if (blockIdx.x > 0) {
    const int64_t i = (int64_t)(blockIdx.x - 1) * 1024 + threadIdx.x;
    if (i < nblocks) mxfp8_block(x, i, elems, scales);
    return;
  }
  build_plan(offsets, E, chunk, hot_ids, n_hot, 1, plan);
}

hipError_t launch_hot_prepare(const int32_t* offsets, int E, int chunk_rows, const int32_t* hot_ids,
                              int n_hot, int32_t* plan, const uint16_t* x, int T, int H, uint8_t* xq,
                              uint8_t* xqs, hipStream_t s) {
  const int64_t nb = (int64_t)T * (H / 32);
  const int blocks = 1 + (int)((nb + 1023) / 1024);
  hot_prepare_kernel<<<blocks, 1024, 0, s>>>(offsets, E, chunk_rows, hot_ids, n_hot, plan, (const uint4*)x,
                                             nb, (uint4*)xq, xqs);
  return hipGetLastError();
}

hipError_t launch_mxfp8_quantize(const uint16_t* x, int64_t rows, int K, uint8_t* elems,
                                 uint8_t* scales, hipStream_t s) {
  const int64_t nb = rows * (K / 32);
  if (nb == 0) return hipSuccess;
  mxfp8_quant_kernel<<<(unsigned)((nb + 255) / 256), 256, 0, s>>>((const uint4*)x, nb, (uint4*)elems, scales);
  return hipGetLastError();
}

// ------------------------------------------------------------------ MXFP4 -> FP8
// Converts n16 chunks of 16 code bytes (32 elements each) and n_sc scale bytes; a block
// works on one matrix of one hot expert.  For the FFN, blockIdx.y = slot within the batch and
// the expert is skipped (no writes) when it has no rows.
struct ConvertJob {
  const uint8_t* codes;
  const uint8_t* scales;
  uint8_t* elems;
  uint8_t* out_scales;
  int64_t n16;        // 16-byte code chunks
  int64_t n_sc;       // scale bytes
  int64_t src_stride, src_sc_stride;  // source bytes per hot expert (0 for a single matrix)
};

__global__ __launch_bounds__(256) void mxfp4_convert_kernel(ConvertJob j1, ConvertJob j2, int two,
                                                            const int32_t* __restrict__ hot_ids,
                                                            const int32_t* __restrict__ counts,
                                                            int n_hot, int E, int b0, int64_t slot_bytes) {
  const int sl = blockIdx.y;
  const int s = b0 + sl;
  if (hot_ids) {
    if (s >= n_hot) return;
    const int he = hot_ids[s];
    if ((unsigned)he >= (unsigned)E || counts[he] == 0) return;  // invalid ids convert nothing
  }
  const bool second = two && blockIdx.z == 1;
  const ConvertJob& J = second ? j2 : j1;
  const uint4* src = (const uint4*)(J.codes + (int64_t)s * J.src_stride);
  uint4* dst = (uint4*)(J.elems + (int64_t)sl * slot_bytes);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < J.n16; i += stride) {
    const uint4 c = src[i];
    uint32_t o[8];
    e2m1x8_to_e4m3(c.x, o[0], o[1]);
    e2m1x8_to_e4m3(c.y, o[2], o[3]);
    e2m1x8_to_e4m3(c.z, o[4], o[5]);
    e2m1x8_to_e4m3(c.w, o[6], o[7]);
    dst[2 * i] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[2 * i + 1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
  const uint8_t* ssrc = J.scales + (int64_t)s * J.src_sc_stride;
  uint8_t* sdst = J.out_scales + (int64_t)sl * slot_bytes;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < J.n_sc; i += stride) sdst[i] = ssrc[i];
}

hipError_t launch_mxfp4_to_fp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int K,
                               uint8_t* elems, uint8_t* out_scales, hipStream_t s) {
  ConvertJob j{codes, scales, elems, out_scales, rows * (K / 32), rows * (K / 32), 0, 0};
  if (j.n16 == 0) return hipSuccess;
  const int64_t want = (j.n16 + 255) / 256;
  const unsigned gx = (unsigned)(want < 4096 ? want : 4096);
  mxfp4_convert_kernel<<<dim3(gx, 1, 1), 256, 0, s>>>(j, j, 0, nullptr, nullptr, 0, 0, 0, 0);
  return hipGetLastError();
}

// ------------------------------------------------------------------ FP8 grouped GEMM
constexpr int kF8BM = 128, kF8BN = 256, kF8BK = 128, kF8Threads = 512;
// One K step of the workgroup tile in LDS: A (token) and B (weight) rows of 128 bytes whose
// 16-byte chunks sit XOR-swizzled by the row (chunk c of row r at position c ^ ((r / 2) % 8):
// the LDS serves a 128-bit read 16 lanes at a time across 64 banks, i.e. two 128-byte rows, so
// one chunk read from 16 consecutive rows hits 16 different bank groups), then the e8m0 scales
// (4 bytes per row), then a pad that the idle lanes' scale loads write into.
constexpr int kF8TileA = kF8BM * kF8BK;             // 16 KB
constexpr int kF8TileB = kF8BN * kF8BK;             // 32 KB
constexpr int kF8SclA = kF8BM * (kF8BK / 32);       // 512 B
constexpr int kF8SclB = kF8BN * (kF8BK / 32);       // 1 KB
constexpr int kF8Pad = 2 * 256;                     // waves 6, 7: one 256-byte scale load each
constexpr int kF8Stage = kF8TileA + kF8TileB + kF8SclA + kF8SclB + kF8Pad;  // 50,688 B
constexpr int kF8Loads = 7;  // direct loads per wave and step: 2 A, 4 B, 1 scale

__device__ __forceinline__ f32x16_t mfma_scale_32x32x64_fp8(i32x8_t a, i32x8_t b, f32x16_t c, uint32_t sa,
                                                           uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, (int)sa, 0, (int)sb);
}

typedef __attribute__((address_space(3))) void lds8_void;

// The operands of one 64-k sub-step for one wave: its two A and two B 32-row tiles (32 bytes
// per lane) and their scale bytes.
struct F8Sub {
  i32x8_t a[2], b[2];
  uint32_t sa[2], sb[2];
};

// Work item = (row tile of <= 128 grouped rows of one hot expert, column tile of 256 weight
// rows); items of experts outside this batch's slots are skipped.  8 waves (2 x 4), each a
// 64 x 64 tile of 2 x 2 MFMA 32x32x64 tiles; one workgroup per CU.  K steps of 128 run through
// a ring of three LDS stages filled by direct global -> LDS loads (no registers, no LDS store
// instructions), two steps ahead.  At step kb a wave waits for its own loads of stage kb+1 and
// for its reads of stage kb, meets the others at one barrier (stage kb+1 is complete and stage
// kb's buffer is free), refills that buffer with stage kb+3, reads stage kb+1's operands into
// its second register set and then issues stage kb's MFMAs: the LDS reads of the next step run
// while the matrix cores work on this one.  The 128 x 256 tile reads 384 bytes of operands from
// L2 per k for 64 K MACs.
// The ring runs on across a workgroup's tasks: the last three steps of a task load the first
// three stages of the next one (whose perm entries were fetched when the task began), so the
// next task starts on stages already in LDS while this one's epilogue runs.  Every step issues
// exactly 7 direct loads per wave (a step with nothing left to load re-reads the last stage,
// which nobody reads), which is what the vmcnt(7) of each step's wait counts on.
//   FC1: A = MXFP8 x rows gathered by perm / ktop; B = W1 image of the slot (rows [0, 2I));
//        column tile n: wave column wn holds gate rows 128n + 32wn + [0,32) and up rows
//        I + 128n + 32wn + [0,32); epilogue h = silu(gate) * up, MXFP8 per 32 columns -> hq.
//   FC2: A = hq rows r0 ..; B = W2 image (rows [0, H)); epilogue y (fp32).
// MODE = (K / 128) % 3 when K / 128 >= 3 (it fixes the ring buffer of every step at compile
// time), 3 for K / 128 < 3 (no prefetch across tasks).
template <int FC, int MODE>
__global__ __launch_bounds__(kF8Threads, 1) void fp8_gemm_kernel(
    const int32_t* __restrict__ plan, int b0, int S, const uint8_t* __restrict__ slots,
    int64_t slot_bytes, int64_t w_off, int64_t ws_off, int rows_per_expert, int K, int width,
    int ktop, const uint8_t* __restrict__ asrc, const uint8_t* __restrict__ ascale,
    const int32_t* __restrict__ perm, int64_t a_rows, void* __restrict__ out,
    uint8_t* __restrict__ out_scale) {
  // three stages as separate objects, so that waiting for one stage's loads does not wait for
  // the others' (gfx950 has 160 KB of LDS per CU)
  __shared__ __align__(16) uint8_t st0[kF8Stage];
  __shared__ __align__(16) uint8_t st1[kF8Stage];
  __shared__ __align__(16) uint8_t st2[kF8Stage];
  const int tid = threadIdx.x, lane = wave_lane(), w = tid / kWave;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index as a uniform value
  const int wm = w & 1, wn = w >> 1, hl = lane >> 5, r32 = lane & 31;  // 2 x 4 waves
  const int n_items = plan[0];
  const int4* items = reinterpret_cast<const int4*>(plan + 4);
  const int n_ntiles = FC == 1 ? width / (kF8BN / 2) : rows_per_expert / kF8BN;
  const int total = n_items * n_ntiles;
  const int nk = K / kF8BK, kb32 = K / 32;
  // direct loads: round u of wave w fills LDS bytes [1024 (8u + w), +1024) of a tile, i.e.
  // rows 8 (8u + w) + lane / 8, position lane % 8, which holds chunk (lane % 8) ^ ((row / 2) % 8)
  const int prow = lane >> 3, ppos = lane & 7;
  // scale loads (4 bytes per lane = one row's four e8m0 scales of the step): waves 0, 1 the A
  // rows 64w + lane, waves 2..5 the B rows 64(w - 2) + lane, waves 6, 7 nothing (kOffNone)
  const bool a_side = wu < 2;
  const int sdst = kF8TileA + kF8TileB + 256 * w;  // LDS offset of this wave's scale load

  // first task at or after t (stride gridDim.x) whose expert has a slot in this batch, or total
  auto next_task = [&](int t) {
    for (; t < total; t += gridDim.x) {
      const int sl = items[t / n_ntiles].w - b0;
      if (sl >= 0 && sl < S) break;
    }
    return t;
  };
  // B rows of the tile (LDS row j -> weight row) of column tile nt
  auto wrow_of = [&](int nt, int j) {
    if (FC == 1) {
      const int jw = j >> 6, jj = j & 63;
      return jj < 32 ? 128 * nt + 32 * jw + jj : width + 128 * nt + 32 * jw + (jj - 32);
    }
    return kF8BN * nt + j;
  };

  // The task whose stages are being loaded: its buffer resources and this lane's offsets.
  buf_rsrc ra, ras, rb, rbs;
  uint32_t aoff[2], boff[4], soff;
  // A task: index, column tile, first grouped row, rows, slot; for FC1 also the perm entries of
  // this lane's two A rows and of its scale row (loaded by every lane, clamped into the item).
  struct Task {
    int t, nt, r0, nrows, slot;
    int praw[3];
  };
  auto begin = [&](Task& T, int t) {
    const int item = t / n_ntiles;
    const int4 itm = items[item];
    T.t = t;
    T.nt = t - item * n_ntiles;
    T.r0 = itm.y;
    T.nrows = itm.z;
    T.slot = itm.w - b0;
    if (FC == 1) {
#pragma unroll
      for (int u = 0; u < 2; ++u) T.praw[u] = perm[T.r0 + min(8 * (8 * u + w) + prow, T.nrows - 1)];
      T.praw[2] = perm[T.r0 + min(64 * (w & 1) + lane, T.nrows - 1)];
    }
  };
  // makes T the task being loaded
  auto finish = [&](const Task& T) {
    const uint8_t* img = slots + (int64_t)T.slot * slot_bytes;
    rb = make_rsrc(img + w_off, (uint32_t)rows_per_expert * K);
    rbs = make_rsrc(img + ws_off, (uint32_t)rows_per_expert * kb32);
    if (FC == 1) {
      ra = make_rsrc(asrc, (uint32_t)(a_rows * K));
      ras = make_rsrc(ascale, (uint32_t)(a_rows * kb32));
    } else {
      ra = make_rsrc(asrc + (int64_t)T.r0 * K, (uint32_t)T.nrows * K);
      ras = make_rsrc(ascale + (int64_t)T.r0 * kb32, (uint32_t)T.nrows * kb32);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = 8 * (8 * u + w) + prow;
      const uint32_t arow = FC == 1 ? (uint32_t)(T.praw[u] / ktop) : (uint32_t)r;
      aoff[u] = r < T.nrows ? arow * (uint32_t)K + 16u * (uint32_t)(ppos ^ ((r >> 1) & 7)) : kOffNone;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = 8 * (8 * u + w) + prow;
      boff[u] = (uint32_t)wrow_of(T.nt, j) * K + 16u * (uint32_t)(ppos ^ ((j >> 1) & 7));
    }
    soff = kOffNone;
    if (w < 2) {
      const int r = 64 * w + lane;
      if (r < T.nrows) soff = (FC == 1 ? (uint32_t)(T.praw[2] / ktop) : (uint32_t)r) * (uint32_t)kb32;
    } else if (w < 6) {
      soff = (uint32_t)wrow_of(T.nt, 64 * (w - 2) + lane) * (uint32_t)kb32;
    }
  };

  auto stage_ptr = [&](int s) -> uint8_t* { return s == 0 ? st0 : (s == 1 ? st1 : st2); };
  // the loads of step kb of the task being loaded into stage buffer s
  auto load_stage = [&](int s, int kb) {
    uint8_t* st = stage_ptr(s);
    const uint32_t ko = (uint32_t)kb * kF8BK;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds8_void*)(st + 1024 * (8 * u + wu)), 16, (int)aoff[u],
                                               (int)ko, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds8_void*)(st + kF8TileA + 1024 * (8 * u + wu)), 16,
                                               (int)boff[u], (int)ko, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_side ? ras : rbs, (lds8_void*)(st + sdst), 4, (int)soff,
                                             (int)(ko / 32), 0, 0);
  };
  // this wave's operands of sub-step kk of a step from stage buffer s.  Tile rows 64 wm + 32 t
  // + r32 have (row / 2) % 8 == (r32 / 2) % 8, so the swizzled position of chunk c is the same
  // for every tile: per lane four chunk offsets (c = hl, 2 + hl, 4 + hl, 6 + hl) and a row base,
  // the rest are instruction offsets.
  uint32_t cofs[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cofs[j] = 16u * (uint32_t)((2 * j + hl) ^ ((r32 >> 1) & 7));
  const uint32_t abase = 128u * (uint32_t)(64 * wm + r32), bbase = 128u * (uint32_t)(64 * wn + r32);
  const uint32_t sabase = 4u * (uint32_t)(64 * wm + r32) + hl, sbbase = 4u * (uint32_t)(64 * wn + r32) + hl;
  auto read_sub = [&](F8Sub& o, int s, int kk) {
    const uint8_t* la = stage_ptr(s);
    const uint8_t* lb = la + kF8TileA;
    const uint8_t* lsa = lb + kF8TileB;
    const uint8_t* lsb = lsa + kF8SclA;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(la + abase + cofs[2 * kk] + 4096 * t);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(la + abase + cofs[2 * kk + 1] + 4096 * t);
      const u32x4 b0_ = *reinterpret_cast<const u32x4*>(lb + bbase + cofs[2 * kk] + 4096 * t);
      const u32x4 b1_ = *reinterpret_cast<const u32x4*>(lb + bbase + cofs[2 * kk + 1] + 4096 * t);
      o.a[t] = i32x8_t{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      o.b[t] = i32x8_t{(int)b0_[0], (int)b0_[1], (int)b0_[2], (int)b0_[3], (int)b1_[0], (int)b1_[1], (int)b1_[2],
                       (int)b1_[3]};
      o.sa[t] = lsa[sabase + 128 * t + 2 * kk];
      o.sb[t] = lsb[sbbase + 128 * t + 2 * kk];
    }
  };

  f32x16_t acc[2][2];
  // The MFMA builtins are pure, so the optimizer may sink them past the barriers and reads
  // that follow (and keep every operand live until then): an empty volatile asm that reads the
  // accumulators keeps each sub-step's MFMAs where they are issued.
  // FC1 takes the weight tile as the matrix cores' A operand, so that a lane's 16 results are
  // 16 channels of one token row (the MXFP8 block of h is then 16 values in each of two lanes);
  // FC2 keeps the token tile as A (a lane holds one column of 16 rows of y).
  auto mfma_sub = [&](const F8Sub& o) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[a][b] = FC == 1 ? mfma_scale_32x32x64_fp8(o.b[b], o.a[a], acc[a][b], o.sb[b], o.sa[a])
                            : mfma_scale_32x32x64_fp8(o.a[a], o.b[b], acc[a][b], o.sa[a], o.sb[b]);
    asm volatile("" ::"v"(acc[0][0]), "v"(acc[0][1]), "v"(acc[1][0]), "v"(acc[1][1]));
  };

  const int t_first = next_task(blockIdx.x);
  if (t_first >= total) return;  // uniform over the block
  Task cur, nxt;
  begin(cur, t_first);
  finish(cur);

  // Step kb (stage kb in buffer D; sub-step 0's operands already in s0):
  //   read sub-step 1 into s1; MFMAs of sub-step 0;
  //   wait for this wave's loads of stage kb+1 and its reads of stage kb; barrier: stage kb+1
  //   is complete and nobody reads buffer D any more; load stage kl of the task being loaded
  //   into D (kb+3 of this task, 0..2 of the next one, or a copy of the last stage);
  //   read sub-step 0 of step kb+1 into s0 (unless kb is the last step); MFMAs of sub-step 1.
  F8Sub s0, s1;
  auto step = [&](auto D_, int kb, int kl, bool read_next) {
    constexpr int D = decltype(D_)::value;
    read_sub(s1, D, 1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_sub(s0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((kF8Loads & 15) | 0x70 | ((kF8Loads >> 4) << 14));  // vmcnt(7), lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    load_stage(D, kl);
    if (read_next) read_sub(s0, (D + 1) % 3, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_sub(s1);
    __builtin_amdgcn_sched_barrier(0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // the first three stages of the task being loaded into buffers P, P+1, P+2, then the wait for
  // stage 0 (every wave)
  auto prologue = [&](auto P_) {
    constexpr int P = decltype(P_)::value;
    load_stage(P, 0);
    load_stage((P + 1) % 3, min(1, nk - 1));
    load_stage((P + 2) % 3, min(2, nk - 1));
    __builtin_amdgcn_s_waitcnt((2 * kF8Loads & 15) | 0x70 | 0xF00 | (((2 * kF8Loads) >> 4) << 14));  // vmcnt(14)
    asm volatile("s_barrier" ::: "memory");
  };
  // The K loop of the current task (K / 128 >= 3), its stage 0 in buffer P and already in LDS:
  // steps whose kb+3 is still in the task, then three steps that load the next task's stages
  // 0..2 (pf) or copies.
  auto run = [&](auto P_, bool pf) {
    constexpr int P = decltype(P_)::value;
    using IP0 = std::integral_constant<int, P>;
    using IP1 = std::integral_constant<int, (P + 1) % 3>;
    using IP2 = std::integral_constant<int, (P + 2) % 3>;
    constexpr int Q = (P + MODE) % 3;  // buffer of the first of the last three steps
    using IQ0 = std::integral_constant<int, Q>;
    using IQ1 = std::integral_constant<int, (Q + 1) % 3>;
    using IQ2 = std::integral_constant<int, (Q + 2) % 3>;
    read_sub(s0, P, 0);
    int kb = 0;
    for (; kb + 6 <= nk; kb += 3) {
      step(IP0{}, kb, kb + 3, true);
      step(IP1{}, kb + 1, kb + 4, true);
      step(IP2{}, kb + 2, kb + 5, true);
    }
    if (MODE >= 1) step(IP0{}, kb, kb + 3, true);  // nk - 3 - kb == MODE steps remain before the last three
    if (MODE >= 2) step(IP1{}, kb + 1, kb + 4, true);
    kb = nk - 3;
    if (pf) finish(nxt);  // the loads below are the next task's
    step(IQ0{}, kb, pf ? 0 : nk - 1, true);
    step(IQ1{}, kb + 1, pf ? 1 : nk - 1, true);
    step(IQ2{}, kb + 2, pf ? 2 : nk - 1, false);
  };
  // K / 128 < 3: the task loads its own stages into buffers 0..2
  auto run_small = [&]() {
    prologue(I0{});
    read_sub(s0, 0, 0);
    step(I0{}, 0, nk - 1, nk > 1);
    if (nk > 1) step(I1{}, 1, nk - 1, false);
  };

  // One task (its stage 0 in buffer P, or K / 128 < 3); returns false after the last one.
  auto task = [&](auto P_) -> bool {
    const int tn = next_task(cur.t + (int)gridDim.x);
    const bool has_next = tn < total, pf = MODE < 3 && has_next;
    if (has_next) begin(nxt, tn);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
    if (MODE == 3)
      run_small();
    else
      run(P_, pf);
    // No LDS is read past the last step's barrier, so the next task's loads can land while the
    // epilogue runs.

    // ---- epilogue
    const int nt_i = cur.nt, r0 = cur.r0, nrows = cur.nrows;
    if (FC == 1) {
      // acc[a][0] (gate) and acc[a][1] (up), element v: token row 64 wm + 32 a + r32 of the
      // tile, channel 128 nt + 32 wn + 8 (v / 4) + 4 hl + v % 4.  The channels 128 nt + 32 wn +
      // [0, 32) are one MXFP8 block of h, held by lanes r32 and r32 + 32.
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float hv[16];
        uint32_t m = 0;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float gt = acc[a][0][v], up = acc[a][1][v];
          hv[v] = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;  // silu(gate) * up
          m = max(m, __float_as_uint(hv[v]) & 0x7FFFFFFFu);
        }
        m = max(m, (uint32_t)__shfl_xor((int)m, 32));
        const int shared = mx_shared_exp(m ? floor_log2_f32(m) : 0, m == 0);
        const int row = 64 * wm + 32 * a + r32;
        if (row < nrows) {
          const int64_t r = (int64_t)(r0 + row);
          const int c0 = 128 * nt_i + 32 * wn;
          uint32_t* dst = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(out) + r * width + c0 + 4 * hl);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dst[2 * q] = e4m3x4_scaled(hv[4 * q], hv[4 * q + 1], hv[4 * q + 2], hv[4 * q + 3], shared);
          if (hl == 0) out_scale[r * (width / 32) + c0 / 32] = (uint8_t)(shared + 127);
        }
      }
    } else {
      // y through a buffer resource that spans the item's nrows rows: the rows past the item
      // are dropped by its bound (no test per value).  y is read once, by the combine:
      // non-temporal stores (aux bit 1) keep it from displacing the weights and h in the caches
      // (FC2 -5 % at 32K rows)
      const buf_rsrc ro = make_rsrc(reinterpret_cast<float*>(out) + (int64_t)r0 * width,
                                    (uint32_t)nrows * (uint32_t)width * 4u);
      const uint32_t vo = ((uint32_t)(64 * wm + 4 * hl) * (uint32_t)width + (uint32_t)(kF8BN * nt_i + 64 * wn + r32)) * 4u;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t off = vo + (uint32_t)(32 * a + 8 * (i >> 2) + (i & 3)) * (uint32_t)width * 4u;
#pragma unroll
          for (int b = 0; b < 2; ++b)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[a][b][i]), ro, (int)(off + 128u * b), 0, 2);
        }
      }
    }
    if (!has_next) return false;
    cur = nxt;
    if (!pf) finish(cur);
    return true;
  };

  // With K / 128 = 3q + MODE the next task's stage 0 lands in buffer (P + MODE) % 3, so the
  // tasks of a workgroup cycle through the buffers 0, MODE, 2 MODE (mod 3); the loop is unrolled
  // over that cycle so that every step's buffers are known at compile time.
  if (MODE == 3) {
    while (task(I0{})) {
    }
  } else {
    prologue(I0{});
    constexpr int P1 = MODE % 3, P2 = (2 * MODE) % 3;
    for (;;) {
      if (!task(I0{})) break;
      if (MODE == 0) continue;
      if (!task(std::integral_constant<int, P1>{})) break;
      if (!task(std::integral_constant<int, P2>{})) break;
    }
  }
  // the loads past the end (copies of the last stage) land before the workgroup's LDS is freed
  __builtin_amdgcn_s_waitcnt(0xC07F & ~0xC00F);  // vmcnt(0), lgkmcnt(0)
}

// ------------------------------------------------------------------ launchers
HotLayout hot_layout(int H, int I) {
  HotLayout L;
  const int64_t w1 = (int64_t)2 * I * H, w2 = (int64_t)H * I;
  auto al = [](int64_t v) { return (v + 255) & ~(int64_t)255; };
  L.w1_off = 0;
  L.w1s_off = al(w1);
  L.w2_off = L.w1s_off + al(w1 / 32);
  L.w2s_off = L.w2_off + al(w2);
  L.slot_bytes = L.w2s_off + al(w2 / 32);
  return L;
}

hipError_t launch_hot_convert(const HotWeights& hw, int H, int I, const int32_t* counts, int b0,
                              int S, uint8_t* slots, hipStream_t s) {
  const HotLayout L = hot_layout(H, I);
  const int64_t w1 = (int64_t)2 * I * H, w2 = (int64_t)H * I;
  ConvertJob j1{hw.w1_codes, hw.w1_scales, slots + L.w1_off, slots + L.w1s_off, w1 / 32, w1 / 32,
                w1 / 2, w1 / 32};
  ConvertJob j2{hw.w2_codes, hw.w2_scales, slots + L.w2_off, slots + L.w2s_off, w2 / 32, w2 / 32,
                w2 / 2, w2 / 32};
  const int nb = hw.n_hot - b0 < S ? hw.n_hot - b0 : S;
  if (nb <= 0) return hipSuccess;
  // ~64 K threads per matrix and slot
  mxfp4_convert_kernel<<<dim3(256, nb, 2), 256, 0, s>>>(j1, j2, 1, hw.hot_ids, counts, hw.n_hot, hw.E, b0,
                                                        L.slot_bytes);
  return hipGetLastError();
}

template <int FC>
static hipError_t launch_fp8(const int32_t* plan, int b0, int S, const uint8_t* slots, int64_t slot_bytes,
                             int64_t w_off, int64_t ws_off, int rows, int K, int width, int ktop,
                             const uint8_t* asrc, const uint8_t* ascale, const int32_t* perm,
                             int64_t a_rows, int64_t tasks, void* out, uint8_t* out_scale,
                             hipStream_t s) {
  const int64_t cap = 256;  // one workgroup per CU
  const int grid = (int)(tasks < cap ? (tasks > 0 ? tasks : 1) : cap);
  const int nk = K / kF8BK;
  auto go = [&](auto kern) {
    kern<<<grid, kF8Threads, 0, s>>>(plan, b0, S, slots, slot_bytes, w_off, ws_off, rows, K, width, ktop, asrc,
                                     ascale, perm, a_rows, out, out_scale);
  };
  if (nk < 3)
    go(fp8_gemm_kernel<FC, 3>);
  else if (nk % 3 == 0)
    go(fp8_gemm_kernel<FC, 0>);
  else if (nk % 3 == 1)
    go(fp8_gemm_kernel<FC, 1>);
  else
    go(fp8_gemm_kernel<FC, 2>);
  return hipGetLastError();
}

hipError_t launch_hot_fc1(int H, int I, int k, int T, const int32_t* hot_plan, int max_items, int b0,
                          int S, const uint8_t* slots, const uint8_t* xq, const uint8_t* xqs,
                          const int32_t* perm, uint8_t* hq, uint8_t* hqs, hipStream_t s) {
  const HotLayout L = hot_layout(H, I);
  return launch_fp8<1>(hot_plan, b0, S, slots, L.slot_bytes, L.w1_off, L.w1s_off, 2 * I, H, I, k, xq, xqs,
                       perm, T, (int64_t)max_items * (I / (kF8BN / 2)), hq, hqs, s);
}

hipError_t launch_hot_fc2(int H, int I, int64_t R, const int32_t* hot_plan, int max_items, int b0,
                          int S, const uint8_t* slots, const uint8_t* hq, const uint8_t* hqs,
                          float* y, hipStream_t s) {
  const HotLayout L = hot_layout(H, I);
  return launch_fp8<2>(hot_plan, b0, S, slots, L.slot_bytes, L.w2_off, L.w2s_off, H, I, H, 1, hq, hqs,
                       nullptr, R, (int64_t)max_items * (H / kF8BN), y, nullptr, s);
}

}  // namespace bitmoe
