// Expert FFN for prefill-sized groups: a grouped GEMM on the matrix cores with the low-bit
// codebook weights decoded into bf16 tiles in LDS.
//
// [Moet-README] release notes of -r23: the prefill MoE is FC1 + SwiGLU, then FC2, over the
// routed rows of each expert.  [Moet-QA]: 2-bit codes on {-4,-1,1,4}, a bf16 scale per 32
// along K.  [Strata-R9700] path 6: 3-bit codes on eight levels, an e4m3 scale / 64 per 64.
//
// Work item = (row tile of <= 128 grouped rows of one expert, column tile of 256 weight rows).
// A workgroup of 8 waves (2 x 4) computes the 128 x 256 tile with v_mfma_f32_32x32x16_bf16,
// each wave 64 x 64 (2 x 2 MFMA tiles).  Per 64-wide K step the workgroup loads the token rows
// (16 KB, gathered) and the packed codes of its 256 weight rows, decodes the codes to exact
// bf16 into LDS (the same decode as the streaming kernels, lowbit_fmt.h), and runs 16 MFMAs
// per wave; LDS is double buffered and the global loads run two steps ahead.  The token rows
// are the traffic that bounds this kernel (the weights are 2-3 bits), so the tile is wide in
// N, and the column tiles of one item are given to the workgroups of one XCD (workgroups are
// dispatched to the 8 XCDs round robin), so its token rows are fetched into that XCD's L2 once.
// Token operand and decoded weights share the format's k-slot order: x comes permuted from the
// prepare kernel and FC1 writes h permuted, so A and B always agree.
//   FC1 column tile n: wave column wn holds gate rows 128n + 32wn + [0,32) and the up rows
//       I + 128n + 32wn + [0,32) as its two MFMA column tiles, so gate and up of one h column
//       sit in the same lane and SwiGLU is applied in the epilogue (h stored bf16).
//   FC2 column tile n: weight rows 256n + [0,256); the epilogue stores y (fp32).
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "lowbit_fmt.h"

namespace bitmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// D(32x32, f32) += A(32x16) * B(16x32).  Lane l supplies A row l%32 and B column l%32 for
// k = 8*(l/32) .. +7; it receives D[8*(j/4) + 4*(l/32) + j%4][l%32] in register j.
__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int kBM = 128, kBN = 256, kBK = 64, kThreads = 512;
constexpr int kLdsRow = kBK + 8;                   // bf16 per LDS row (16 B of padding)
constexpr int kATile = kBM * kLdsRow;              // A tile (bf16 elements)
constexpr int kBufElems = (kBM + kBN) * kLdsRow;   // A + B tiles of one buffer
constexpr int kGemmLds = 2 * kBufElems * 2;        // 2 buffers x bf16 = 110,592 B
constexpr int kGemmGrid = 256;                     // one workgroup per CU, 32 per XCD

template <class F, int FC>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int rows_per_expert,
    int K, int width, int ktop, const uint16_t* __restrict__ asrc, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ plan, uint32_t asrc_bytes, void* __restrict__ out) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, lane = wave_lane(), w = tid / kWave;
  const int wm = w & 1, wn = w >> 1;
  const int n_items = plan[0];
  const int4* items = reinterpret_cast<const int4*>(plan + 4);
  const int n_ntiles = FC == 1 ? width / 128 : rows_per_expert / kBN;
  const uint32_t cbr = F::code_bytes((uint32_t)K), sbr = F::scale_bytes((uint32_t)K);
  const int nk = K / kBK;
  // XCD-aware order: the workgroups of XCD x (blockIdx % 8, for a grid that is a multiple of 8)
  // take the items x, x + 8, ..., all column tiles of an item in a row
  const int xcd = blockIdx.x & 7, nb_x = gridDim.x >> 3, lb = blockIdx.x >> 3;
  const int items_x = n_items > xcd ? (n_items - xcd + 7) >> 3 : 0;
  const int total_x = items_x * n_ntiles;

  for (int p = lb; p < total_x; p += nb_x) {
    const int item = xcd + 8 * (p / n_ntiles), nt_i = p % n_ntiles;
    const int4 itm = items[item];
    const int e = itm.x, r0 = itm.y, nrows = itm.z;
    const size_t ebase = (size_t)e * rows_per_expert;

    // ---- per-thread load assignments for this tile (uniform buffer bases, per-lane offsets)
    // A: 128 rows x 8 chunks of 16 B per K step; thread owns rows (tid >> 3) + 64 u (u = 0, 1),
    //    chunk tid & 7.  FC1 gathers token rows of x (all of x is addressable); FC2 reads h
    //    rows r0.. of this tile (based at r0: h may reach 2 GiB).
    const buf_rsrc ra = FC == 1 ? make_rsrc(asrc, asrc_bytes)
                                : make_rsrc(asrc + (size_t)r0 * K, (uint32_t)nrows * K * 2u);
    uint32_t aoff[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = (tid >> 3) + 64 * u;
      const int rr = min(r, nrows - 1);
      const uint32_t tok = FC == 1 ? (uint32_t)(perm[r0 + rr] / ktop) : (uint32_t)rr;
      aoff[u] = r < nrows ? (tok * (uint32_t)K + 8u * (tid & 7)) * 2u : kOffNone;
    }
    // B: weight row j = tid >> 1 of the tile, half h = tid & 1 of its 64 codes (32 codes).
    const int j = tid >> 1, hsel = tid & 1;
    int wrow;
    if (FC == 1) {
      const int jw = j >> 6, jj = j & 63;  // wave column, position in it
      wrow = (jj < 32 ? 128 * nt_i + 32 * jw + jj : width + 128 * nt_i + 32 * jw + (jj - 32));
    } else {
      wrow = kBN * nt_i + j;
    }
    const buf_rsrc rc = make_rsrc(codes + ebase * cbr, (uint32_t)rows_per_expert * cbr);
    const buf_rsrc rs = make_rsrc(scales + ebase * sbr, (uint32_t)rows_per_expert * sbr);
    const uint32_t coff = (uint32_t)wrow * cbr + F::code_bytes(32u * hsel);
    // 2-bit: the half's own bf16 scale; 3-bit: the step's one scale byte (shared by both halves)
    const uint32_t soff = (uint32_t)wrow * sbr + (F::kId == W2Fmt::kId ? 2u * hsel : 0u);
    const uint32_t cstep = F::code_bytes(kBK), sstep = F::scale_bytes(kBK);

    // register staging of K steps, two deep: the loads of step kb + 2 are issued while step kb
    // is computed from LDS and step kb + 1 waits in registers to be stored
    struct Staged {
      u32x4 a[2];
      uint32_t c[F::kFieldWords];
      uint32_t s;
    };
    Staged stg[2];
    auto load_step = [&](Staged& g, int kb) {
#pragma unroll
      for (int u = 0; u < 2; ++u) g.a[u] = buf_load16(ra, aoff[u] + (uint32_t)kb * kBK * 2u);
      const uint32_t co = coff + (uint32_t)kb * cstep, so = soff + (uint32_t)kb * sstep;
      const uint64_t c01 = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rc, (int)co, 0, 0));
      g.c[0] = (uint32_t)c01;
      g.c[1] = (uint32_t)(c01 >> 32);
      if constexpr (F::kFieldWords == 3) g.c[2] = buf_load4(rc, co + 8u);
      if constexpr (F::kId == W2Fmt::kId)
        g.s = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)so, 0, 0);
      else
        g.s = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, (int)so, 0, 0);
    };
    auto store_a = [&](const Staged& g, int buf) {
      uint16_t* la = lds + buf * kBufElems;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = (tid >> 3) + 64 * u;
        *reinterpret_cast<u32x4*>(la + r * kLdsRow + 8 * (tid & 7)) = g.a[u];
      }
    };
    // operand op (0..3) of the thread's 32 codes -> its 8 slots of the B tile
    auto store_b = [&](const Staged& g, const typename F::Tab& tab, int buf, int op) {
      uint16_t* dst = lds + buf * kBufElems + kATile + j * kLdsRow + 32 * hsel;
      *reinterpret_cast<u32x4*>(dst + 8 * op) = F::decode32(g.c, tab, op);
    };
    auto store_step = [&](const Staged& g, int buf) {
      store_a(g, buf);
      const typename F::Tab tab = F::table32(g.s);
#pragma unroll
      for (int op = 0; op < 4; ++op) store_b(g, tab, buf, op);
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    // one K step from LDS buffer P; staging slot P is refilled with step kb + 2, and step kb + 1
    // (slot P^1) is stored into the other LDS buffer in quarters between this step's MFMA
    // groups, so the decode's VALU work overlaps the matrix cores.  The operands of sub-step
    // kk + 1 are read from LDS before the MFMAs of kk.  Loads are unconditional (clamped).
    auto iter = [&](auto P_, int kb) {
      constexpr int P = decltype(P_)::value;
      load_step(stg[P], min(kb + 2, nk - 1));
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this step's LDS reads
      const uint16_t* la = lds + P * kBufElems;
      const uint16_t* lbm = la + kATile;
      const bool more = kb + 1 < nk;
      u32x4 av[2][2], bv[2][2];
      auto read_ops = [&](int kk, u32x4* a_, u32x4* b_) {
        const int kof = 16 * kk + 8 * (lane >> 5);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          a_[t] = *reinterpret_cast<const u32x4*>(la + (64 * wm + 32 * t + (lane & 31)) * kLdsRow + kof);
          b_[t] = *reinterpret_cast<const u32x4*>(lbm + (64 * wn + 32 * t + (lane & 31)) * kLdsRow + kof);
        }
      };
      read_ops(0, av[0], bv[0]);
      typename F::Tab tab{};
      if (more) {
        store_a(stg[P ^ 1], P ^ 1);
        tab = F::table32(stg[P ^ 1].s);
      }
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        if (kk + 1 < kBK / 16) read_ops(kk + 1, av[(kk + 1) & 1], bv[(kk + 1) & 1]);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) acc[a][b] = mfma_32x32x16_bf16(av[kk & 1][a], bv[kk & 1][b], acc[a][b]);
        if (more) store_b(stg[P ^ 1], tab, P ^ 1, kk);
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
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
        const int row = 64 * wm + 32 * a + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (row >= nrows) continue;
        const size_t r = (size_t)(r0 + row);
        if (FC == 1) {
          const float gt = acc[a][0][i], up = acc[a][1][i];
          const float hv = __fdividef(gt, 1.0f + __expf(-gt)) * up;
          const int col = 128 * nt_i + 32 * wn + (lane & 31);
          reinterpret_cast<uint16_t*>(out)[r * width + 32 * (col >> 5) + F::pos32(col & 31)] =
              (uint16_t)f32_to_bf16_rne(hv);
        } else {
#pragma unroll
          for (int b = 0; b < 2; ++b)
            reinterpret_cast<float*>(out)[r * width + kBN * nt_i + 64 * wn + 32 * b + (lane & 31)] =
                acc[a][b][i];
        }
      }
    }
  }
}

template <class F, int FC>
static hipError_t launch_gemm(const void* codes, const void* scales, int rows, int K, int width,
                              int ktop, const uint16_t* asrc, const int32_t* perm,
                              const int32_t* plan, uint32_t asrc_bytes, void* out, hipStream_t s) {
  // dynamic LDS above 64 KB must be allowed once per kernel instance
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)gemm_kernel<F, FC>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  gemm_kernel<F, FC><<<kGemmGrid, kThreads, kGemmLds, s>>>((const uint8_t*)codes, (const uint8_t*)scales, rows,
                                                         K, width, ktop, asrc, perm, plan, asrc_bytes, out);
  return hipGetLastError();
}

hipError_t launch_lowbit_gemm_fc1(const LowbitWeights& w, int H, int I, int k, const uint16_t* xp,
                                  const int32_t* perm, const int32_t* plan, int max_items, int T,
                                  uint16_t* hbuf, hipStream_t s) {
  (void)max_items;
  const uint32_t xb = (uint32_t)((size_t)T * H * 2);
  if (w.fmt == W2Fmt::kId)
    return launch_gemm<W2Fmt, 1>(w.w1_codes, w.w1_scales, 2 * I, H, I, k, xp, perm, plan, xb, hbuf, s);
  if (w.fmt == W3Fmt::kId)
    return launch_gemm<W3Fmt, 1>(w.w1_codes, w.w1_scales, 2 * I, H, I, k, xp, perm, plan, xb, hbuf, s);
  return hipErrorInvalidValue;
}

hipError_t launch_lowbit_gemm_fc2(const LowbitWeights& w, int H, int I, int k,
                                  const uint16_t* hbuf, const int32_t* plan, int max_items, int T,
                                  float* y, hipStream_t s) {
  (void)max_items;
  const uint32_t hb = (uint32_t)((size_t)T * k * I * 2);
  if (w.fmt == W2Fmt::kId)
    return launch_gemm<W2Fmt, 2>(w.w2_codes, w.w2_scales, H, I, H, 1, hbuf, nullptr, plan, hb, y, s);
  if (w.fmt == W3Fmt::kId)
    return launch_gemm<W3Fmt, 2>(w.w2_codes, w.w2_scales, H, I, H, 1, hbuf, nullptr, plan, hb, y, s);
  return hipErrorInvalidValue;
}

}  // namespace bitmoe
