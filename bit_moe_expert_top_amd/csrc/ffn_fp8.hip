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

// Maximum over the 32 lanes of each half-wave, in every lane: DPP exchanges within rows of 16
// (xor 1, xor 2, half-row mirror, row mirror), then one ds_swizzle across the two rows of the
// half-wave (bit mode: xor 16) -- instead of five ds_bpermute round trips.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t half_wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  return max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (0x10 << 10) | 0x1F));
}

// ------------------------------------------------------------------ FP8 grouped GEMM
constexpr int kF8BM = 128, kF8BN = 256, kF8BK = 128, kF8Threads = 512;
constexpr int kF8Row = kF8BK + 16;                  // LDS bytes per tile row (16 B of padding)
constexpr int kF8TileA = kF8BM * kF8Row;            // the A (token) tile
constexpr int kF8TileB = kF8BN * kF8Row;            // the B (weight) tile
constexpr int kF8SclA = kF8BM * (kF8BK / 32);       // scale tiles (4 bytes per row)
constexpr int kF8SclB = kF8BN * (kF8BK / 32);
constexpr int kF8Buf = kF8TileA + kF8TileB + kF8SclA + kF8SclB + 16;  // + a dword for idle threads
constexpr int kF8Lds = 2 * kF8Buf;                  // double buffered: 113,696 B

__device__ __forceinline__ f32x16_t mfma_scale_32x32x64_fp8(i32x8_t a, i32x8_t b, f32x16_t c, uint32_t sa,
                                                           uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, (int)sa, 0, (int)sb);
}

// Work item = (row tile of <= 128 grouped rows of one hot expert, column tile of 256 weight
// rows); items of experts outside this batch's slots are skipped.  8 waves (2 x 4), each a
// 64 x 64 tile of 2 x 2 MFMA 32x32x64 tiles; one workgroup per CU; K steps of 128 through
// double-buffered LDS, register-staged two steps ahead.  The 128 x 256 tile reads 384 bytes
// of operands from L2 per k for 64 K MACs (a 128 x 128 tile: 256 for 16 K).  Within a step the
// operands of both 64-k sub-steps are read from LDS (two register sets) before the first
// sub-step's MFMAs, so the second sub-step's LDS latency hides behind them.
//   FC1: A = MXFP8 x rows gathered by perm / ktop; B = W1 image of the slot (rows [0, 2I));
//        column tile n: wave column wn holds gate rows 128n + 32wn + [0,32) and up rows
//        I + 128n + 32wn + [0,32); epilogue h = silu(gate) * up, MXFP8 per 32 columns -> hq.
//   FC2: A = hq rows r0 ..; B = W2 image (rows [0, H)); epilogue y (fp32).
template <int FC>
__global__ __launch_bounds__(kF8Threads, 1) void fp8_gemm_kernel(
    const int32_t* __restrict__ plan, int b0, int S, const uint8_t* __restrict__ slots,
    int64_t slot_bytes, int64_t w_off, int64_t ws_off, int rows_per_expert, int K, int width,
    int ktop, const uint8_t* __restrict__ asrc, const uint8_t* __restrict__ ascale,
    const int32_t* __restrict__ perm, int64_t a_rows, void* __restrict__ out,
    uint8_t* __restrict__ out_scale) {
  __shared__ __align__(16) uint8_t lds8[kF8Lds];  // static: gfx950 has 160 KB of LDS per CU
  const int tid = threadIdx.x, lane = wave_lane(), w = tid / kWave;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the wave index as a uniform value
  const int wm = w & 1, wn = w >> 1, hl = lane >> 5, r32 = lane & 31;  // 2 x 4 waves
  const int n_items = plan[0];
  const int4* items = reinterpret_cast<const int4*>(plan + 4);
  const int n_ntiles = FC == 1 ? width / (kF8BN / 2) : rows_per_expert / kF8BN;
  const int total = n_items * n_ntiles;
  const int nk = K / kF8BK, kb32 = K / 32;

  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    const int item = task / n_ntiles, nt_i = task - item * n_ntiles;
    const int4 itm = items[item];
    const int slot = itm.w - b0;
    if (slot < 0 || slot >= S) continue;  // uniform over the block
    const int r0 = itm.y, nrows = itm.z;
    const uint8_t* img = slots + (int64_t)slot * slot_bytes;

    // A rows: thread owns 16-byte chunks (tid & 7) of rows (tid >> 3) + 32u
    const buf_rsrc ra = FC == 1 ? make_rsrc(asrc, (uint32_t)(a_rows * K))
                                : make_rsrc(asrc + (int64_t)r0 * K, (uint32_t)nrows * K);
    const buf_rsrc ras = FC == 1 ? make_rsrc(ascale, (uint32_t)(a_rows * kb32))
                                 : make_rsrc(ascale + (int64_t)r0 * kb32, (uint32_t)nrows * kb32);
    uint32_t aoff[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = (tid >> 3) + 64 * u;
      aoff[u] = kOffNone;
      if (r < nrows) {
        const uint32_t arow = FC == 1 ? (uint32_t)(perm[r0 + r] / ktop) : (uint32_t)r;
        aoff[u] = arow * (uint32_t)K + 16u * (tid & 7);
      }
    }
    // A scales: threads 0..127 own row tid; B scales: threads 128..255 own row tid - 128
    uint32_t asoff = kOffNone;
    if (tid < 128 && tid < nrows) {
      const uint32_t arow = FC == 1 ? (uint32_t)(perm[r0 + tid] / ktop) : (uint32_t)tid;
      asoff = arow * (uint32_t)kb32;
    }
    // B rows of the tile (LDS row j -> weight row)
    auto wrow_of = [&](int j) {
      if (FC == 1) {
        const int jw = j >> 6, jj = j & 63;
        return jj < 32 ? 128 * nt_i + 32 * jw + jj : width + 128 * nt_i + 32 * jw + (jj - 32);
      }
      return kF8BN * nt_i + j;
    };
    const buf_rsrc rb = make_rsrc(img + w_off, (uint32_t)rows_per_expert * K);
    const buf_rsrc rbs = make_rsrc(img + ws_off, (uint32_t)rows_per_expert * kb32);
    uint32_t boff[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) boff[u] = (uint32_t)wrow_of((tid >> 3) + 64 * u) * K + 16u * (tid & 7);
    const uint32_t bsoff = (tid >= 128 && tid < 384) ? (uint32_t)wrow_of(tid - 128) * kb32 : kOffNone;

    // register staging of K steps, two deep: the loads of step kb + 2 are issued before step kb
    // is computed from LDS; step kb + 1 waits in registers and is stored after the MFMAs
    struct Staged {
      u32x4 a[2], b[4];
      uint32_t s;
    };
    Staged stg[2];
    auto load_step = [&](Staged& g, int kb) {
      const uint32_t ko = (uint32_t)kb * kF8BK;
#pragma unroll
      for (int u = 0; u < 2; ++u) g.a[u] = buf_load16(ra, aoff[u] + ko);
#pragma unroll
      for (int u = 0; u < 4; ++u) g.b[u] = buf_load16(rb, boff[u] + ko);
      // waves 0, 1 (threads 0..127) load the A scales, waves 2, 3 the B scales: the resource is
      // chosen per wave (a per-lane choice of resource makes the compiler loop over both)
      const bool a_side = wu < 2;  // waves 2..5: B scales; waves 6, 7 load nothing (kOffNone)
      g.s = buf_load4(a_side ? ras : rbs, (a_side ? asoff : bsoff) + 4u * kb);
    };
    auto store_step = [&](const Staged& g, int buf) {
      uint8_t* la = lds8 + buf * kF8Buf;
      uint8_t* lb = la + kF8TileA;
      uint8_t* lsa = lb + kF8TileB;
      uint8_t* lsb = lsa + kF8SclA;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        *reinterpret_cast<u32x4*>(la + ((tid >> 3) + 64 * u) * kF8Row + 16 * (tid & 7)) = g.a[u];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<u32x4*>(lb + ((tid >> 3) + 64 * u) * kF8Row + 16 * (tid & 7)) = g.b[u];
      // unconditional stores: threads 384..511 write a scratch dword past the B scales
      *reinterpret_cast<uint32_t*>(tid < 128 ? lsa + 4 * tid : lsb + 4 * min(tid - 128, 256)) = g.s;
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    auto iter = [&](auto P_, int kb) {
      constexpr int P = decltype(P_)::value;
      load_step(stg[P], min(kb + 2, nk - 1));  // unconditional (clamped)
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* la = lds8 + P * kF8Buf;
      const uint8_t* lb = la + kF8TileA;
      const uint8_t* lsa = lb + kF8TileB;
      const uint8_t* lsb = lsa + kF8SclA;
      // operands of sub-step kk (64 k): the A and B tiles of this wave, their scale bytes
      struct Ops {
        i32x8_t a[2], b[2];
        uint32_t sa[2], sb[2];
      };
      auto read_ops = [&](Ops& o, int kk) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int ra_ = 64 * wm + 32 * t + r32, rb_ = 64 * wn + 32 * t + r32;
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(la + ra_ * kF8Row + 64 * kk + 16 * hl);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(la + ra_ * kF8Row + 64 * kk + 32 + 16 * hl);
          const u32x4 b0_ = *reinterpret_cast<const u32x4*>(lb + rb_ * kF8Row + 64 * kk + 16 * hl);
          const u32x4 b1_ = *reinterpret_cast<const u32x4*>(lb + rb_ * kF8Row + 64 * kk + 32 + 16 * hl);
          o.a[t] = i32x8_t{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          o.b[t] = i32x8_t{(int)b0_[0], (int)b0_[1], (int)b0_[2], (int)b0_[3], (int)b1_[0], (int)b1_[1], (int)b1_[2], (int)b1_[3]};
          o.sa[t] = lsa[4 * ra_ + 2 * kk + hl];
          o.sb[t] = lsb[4 * rb_ + 2 * kk + hl];
        }
      };
      static_assert(kF8BK == 128, "two sub-steps per step");
      Ops o0, o1;
      read_ops(o0, 0);
      __builtin_amdgcn_sched_barrier(0);
      read_ops(o1, 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma_scale_32x32x64_fp8(o0.a[a], o0.b[b], acc[a][b], o0.sa[a], o0.sb[b]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma_scale_32x32x64_fp8(o1.a[a], o1.b[b], acc[a][b], o1.sa[a], o1.sb[b]);
      __builtin_amdgcn_sched_barrier(0);  // the store of step kb + 1 after this step's MFMAs
      store_step(stg[P ^ 1], P ^ 1);  // unconditional (at the last step: a clamped reload, unused)
      // LDS writes done, then a bare barrier: step kb + 1 is in LDS for every wave and every wave
      // is done with buffer P.  (A __syncthreads fence would also drain the loads of step kb + 2
      // issued above, which are only needed at the end of the next step.)
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt not waited on
      asm volatile("s_barrier" ::: "memory");
    };

    load_step(stg[0], 0);
    load_step(stg[1], min(1, nk - 1));
    store_step(stg[0], 0);
    __syncthreads();
    for (int kb = 0; kb < nk; kb += 2) {  // nk is even (K is a multiple of 256)
      iter(std::integral_constant<int, 0>{}, kb);
      iter(std::integral_constant<int, 1>{}, kb + 1);
    }

    // ---- epilogue
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 64 * wm + 32 * a + 8 * (i >> 2) + 4 * hl + (i & 3);
        if (FC == 1) {
          const float gt = acc[a][0][i], up = acc[a][1][i];
          const float hv = __fdividef(gt, 1.0f + __expf(-gt)) * up;
          const uint32_t hb = __float_as_uint(hv);
          // MXFP8 over the 32 columns of this row held by the 32 lanes of this half-wave
          uint32_t m = hb & 0x7FFFFFFFu;
          m = half_wave_max_u32(m);
          const int shared = mx_shared_exp(m ? floor_log2_f32(m) : 0, m == 0);
          const uint32_t e = f32_to_e4m3_scaled(hb, shared);
          if (row < nrows) {
            const int64_t r = (int64_t)(r0 + row);
            const int col = 128 * nt_i + 32 * wn + r32;
            reinterpret_cast<uint8_t*>(out)[r * width + col] = (uint8_t)e;
            if (r32 == 0) out_scale[r * (width / 32) + col / 32] = (uint8_t)(shared + 127);
          }
        } else if (row < nrows) {
          const int64_t r = (int64_t)(r0 + row);
#pragma unroll
          for (int b = 0; b < 2; ++b)
            reinterpret_cast<float*>(out)[r * width + kF8BN * nt_i + 64 * wn + 32 * b + r32] = acc[a][b][i];
        }
      }
    }
  }
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
  fp8_gemm_kernel<FC><<<grid, kF8Threads, 0, s>>>(plan, b0, S, slots, slot_bytes, w_off, ws_off, rows, K,
                                                width, ktop, asrc, ascale, perm, a_rows, out, out_scale);
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
