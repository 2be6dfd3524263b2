// Expert FFN for prefill-sized groups: a grouped GEMM on the matrix cores with the 2-bit
// codebook weights decoded into bf16 tiles in LDS.
//
// [Moet-README] release notes of -r23: the prefill MoE is FC1 + SwiGLU, then FC2, over the
// routed rows of each expert.  [Moet-QA] (2-bit experts): codes on {-4,-1,1,4}, one bf16
// scale per 32 weights along K.
//
// Work item = (row tile of <= 128 grouped rows of one expert, column tile of 128 weight rows).
// A workgroup of 4 waves (2 x 2) computes the 128 x 128 tile with v_mfma_f32_32x32x16_bf16,
// each wave 64 x 64 (2 x 2 MFMA tiles).  Per 64-wide K step the workgroup loads the token rows
// (16 KB, gathered) and the packed codes of its 128 weight rows (2 KB + 512 B of scales),
// decodes the codes to bf16 into LDS (the same byte-table decode as the streaming kernels),
// and runs 16 MFMAs per wave; LDS is double buffered so the next step's loads overlap.
// Token operand and decoded weights share the k-slot order of the streaming path (a 4 x 4
// transpose inside every 16 k): x comes permuted from the prepare kernel and FC1 writes h
// permuted, so A and B always agree.
//   FC1 column tile n: wave column wn holds gate rows 64n + 32wn + [0,32) and the up rows
//       I + 64n + 32wn + [0,32) as its two MFMA column tiles, so gate and up of one h column
//       sit in the same lane and SwiGLU is applied in the epilogue (h stored bf16).
//   FC2 column tile n: weight rows 128n + [0,128); the epilogue stores y (fp32).
#include "common.h"
#include "kernels.h"

namespace bitmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// D(32x32, f32) += A(32x16) * B(16x32).  Lane l supplies A row l%32 and B column l%32 for
// k = 8*(l/32) .. +7; it receives D[8*(j/4) + 4*(l/32) + j%4][l%32] in register j.
__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 2-bit group table and decode (identical bit logic to the streaming kernels).
__device__ __forceinline__ void g2_table(uint32_t s16, uint32_t& lut, uint32_t& lb) {
  const uint32_t hb = (s16 >> 8) & 0xFFu;
  lut = ((hb * 0x01010101u) ^ 0x00008080u) + 0x01000001u;
  lb = s16 & 0xFFu;
}
template <int HALF>
__device__ __forceinline__ u32x4 g2_decode(uint32_t w, uint32_t lut, uint32_t lb) {
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
__device__ __forceinline__ int g_kpos16(int f) { return 4 * (f & 3) + (f >> 2); }

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsRow = kBK + 8;                  // bf16 per LDS row (16 B of padding)
constexpr int kTileElems = kBM * kLdsRow;         // one operand tile
constexpr int kGemmLds = 2 * 2 * kTileElems * 2;  // 2 buffers x (A + B) x bf16 = 73,728 B

template <int FC>
__global__ __launch_bounds__(256, 2) void w2_gemm_kernel(
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales, int rows_per_expert,
    int K, int width, int ktop, const uint16_t* __restrict__ asrc, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ plan, uint32_t asrc_bytes, void* __restrict__ out) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, lane = wave_lane(), w = tid / kWave;
  const int wm = w & 1, wn = w >> 1;
  const int n_items = plan[0];
  const int4* items = reinterpret_cast<const int4*>(plan + 4);
  const int n_ntiles = FC == 1 ? width / 64 : rows_per_expert / kBN;
  const int total = n_items * n_ntiles;
  const int wpr = K / 16, spr = K / 32, nk = K / kBK;

  for (int task = blockIdx.x; task < total; task += gridDim.x) {
    const int item = task / n_ntiles, nt_i = task - item * n_ntiles;
    const int4 itm = items[item];
    const int e = itm.x, r0 = itm.y, nrows = itm.z;
    const size_t ebase = (size_t)e * rows_per_expert;

    // ---- per-thread load assignments for this tile (uniform buffer bases, per-lane offsets)
    // A: 128 rows x 8 chunks of 16 B per K step; thread owns chunks tid + 256 u (u = 0..3):
    //    row = (tid >> 3) + 32 u, chunk = tid & 7.  FC1 gathers token rows of x (all of x is
    //    addressable); FC2 reads h rows r0.. of this tile (based at r0: h may reach 2 GiB).
    const buf_rsrc ra = FC == 1 ? make_rsrc(asrc, asrc_bytes)
                                : make_rsrc(asrc + (size_t)r0 * K, (uint32_t)nrows * K * 2u);
    uint32_t aoff[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = (tid >> 3) + 32 * u;
      aoff[u] = kOffNone;
      if (r < nrows) {
        const uint32_t tok = FC == 1 ? (uint32_t)(perm[r0 + r] / ktop) : (uint32_t)r;
        aoff[u] = (tok * (uint32_t)K + 8u * (tid & 7)) * 2u;
      }
    }
    // B: weight row j = tid >> 1 of the tile, half h = tid & 1 of its 64 codes (2 words).
    const int j = tid >> 1, hsel = tid & 1;
    int wrow;
    if (FC == 1) {
      const int jw = j >> 6, jj = j & 63;  // wave column, position in it
      wrow = (jj < 32 ? 64 * nt_i + 32 * jw + jj : width + 64 * nt_i + 32 * jw + (jj - 32));
    } else {
      wrow = kBN * nt_i + j;
    }
    const buf_rsrc rc = make_rsrc(codes + ebase * wpr, (uint32_t)(rows_per_expert * wpr * 4));
    const buf_rsrc rs = make_rsrc(scales + ebase * spr, (uint32_t)(rows_per_expert * spr * 2));
    const uint32_t coff = (uint32_t)(wrow * wpr * 4) + 8u * hsel;
    const uint32_t soff = (uint32_t)(wrow * spr * 2) + 2u * hsel;

    // register staging of one K step
    u32x4 areg[4];
    uint64_t creg;
    uint32_t sreg;
    auto load_step = [&](int kb) {
#pragma unroll
      for (int u = 0; u < 4; ++u) areg[u] = buf_load16(ra, aoff[u] + (uint32_t)kb * kBK * 2u);
      creg = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(
                                              rc, (int)(coff + (uint32_t)kb * 16u), 0, 0));
      sreg = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)(soff + (uint32_t)kb * 4u), 0, 0);
    };
    auto store_step = [&](int buf) {
      uint16_t* la = lds + buf * 2 * kTileElems;
      uint16_t* lbm = la + kTileElems;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = (tid >> 3) + 32 * u;
        *reinterpret_cast<u32x4*>(la + r * kLdsRow + 8 * (tid & 7)) = areg[u];
      }
      uint32_t lut, lb;
      g2_table(sreg & 0xFFFFu, lut, lb);
      uint16_t* dst = lbm + j * kLdsRow + 32 * hsel;
      const uint32_t w0 = (uint32_t)creg, w1 = (uint32_t)(creg >> 32);
      *reinterpret_cast<u32x4*>(dst + 0) = g2_decode<0>(w0, lut, lb);
      *reinterpret_cast<u32x4*>(dst + 8) = g2_decode<1>(w0, lut, lb);
      *reinterpret_cast<u32x4*>(dst + 16) = g2_decode<0>(w1, lut, lb);
      *reinterpret_cast<u32x4*>(dst + 24) = g2_decode<1>(w1, lut, lb);
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    load_step(0);
    store_step(0);
    __syncthreads();
    for (int kb = 0; kb < nk; ++kb) {
      const int buf = kb & 1;
      load_step(min(kb + 1, nk - 1));  // unconditional (the last step reloads itself)
      const uint16_t* la = lds + buf * 2 * kTileElems;
      const uint16_t* lbm = la + kTileElems;
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int kof = 16 * kk + 8 * (lane >> 5);
        u32x4 av[2], bv[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          av[t] = *reinterpret_cast<const u32x4*>(la + (64 * wm + 32 * t + (lane & 31)) * kLdsRow + kof);
          bv[t] = *reinterpret_cast<const u32x4*>(lbm + (64 * wn + 32 * t + (lane & 31)) * kLdsRow + kof);
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b) acc[a][b] = mfma_32x32x16_bf16(av[a], bv[b], acc[a][b]);
      }
      if (kb + 1 < nk) store_step(buf ^ 1);
      __syncthreads();
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
          const int col = 64 * nt_i + 32 * wn + (lane & 31);
          reinterpret_cast<uint16_t*>(out)[r * width + 16 * (col >> 4) + g_kpos16(col & 15)] =
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

static bool g_gemm_attr_set[2] = {false, false};

template <int FC>
static hipError_t launch_gemm(const uint32_t* codes, const uint16_t* scales, int rows, int K,
                              int width, int ktop, const uint16_t* asrc, const int32_t* perm,
                              const int32_t* plan, uint32_t asrc_bytes, int64_t tasks, void* out,
                              hipStream_t s) {
  if (!g_gemm_attr_set[FC - 1]) {
    hipError_t e = hipFuncSetAttribute((const void*)w2_gemm_kernel<FC>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
    if (e != hipSuccess) return e;
    g_gemm_attr_set[FC - 1] = true;
  }
  const int64_t cap = 256 * 2;
  const int grid = (int)(tasks < cap ? (tasks > 0 ? tasks : 1) : cap);
  w2_gemm_kernel<FC><<<grid, 256, kGemmLds, s>>>(codes, scales, rows, K, width, ktop, asrc, perm,
                                                 plan, asrc_bytes, out);
  return hipGetLastError();
}

hipError_t launch_lowbit_gemm_fc1(const LowbitWeights& w, int H, int I, int k, const uint16_t* xp,
                                  const int32_t* perm, const int32_t* plan, int max_items, int T,
                                  uint16_t* hbuf, hipStream_t s) {
  if (w.fmt != 1) return hipErrorInvalidValue;
  return launch_gemm<1>((const uint32_t*)w.w1_codes, (const uint16_t*)w.w1_scales, 2 * I, H, I, k,
                        xp, perm, plan, (uint32_t)((size_t)T * H * 2),
                        (int64_t)max_items * (I / 64), hbuf, s);
}

hipError_t launch_lowbit_gemm_fc2(const LowbitWeights& w, int H, int I, int k,
                                  const uint16_t* hbuf, const int32_t* plan, int max_items, int T,
                                  float* y, hipStream_t s) {
  if (w.fmt != 1) return hipErrorInvalidValue;
  return launch_gemm<2>((const uint32_t*)w.w2_codes, (const uint16_t*)w.w2_scales, H, I, H, 1, hbuf,
                        nullptr, plan, (uint32_t)((size_t)T * k * I * 2),
                        (int64_t)max_items * (H / kBN), y, s);
}

}  // namespace bitmoe
