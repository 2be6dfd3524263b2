// Host-side launchers of the gfx950 kernels (internal to the library; the public C ABI is
// include/bitmoe.h).  Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bitmoe {

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s);

// Rows per block of the multi-block grouping path; R <= kPermuteChunk uses one block.
constexpr int kPermuteChunk = 4096;
size_t permute_ws_bytes(int64_t R, int E);
hipError_t launch_permute(const int32_t* ids, int R, int E, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, void* ws, hipStream_t s);

// Fill with a kernel rather than hipMemsetAsync, so the calls stay graph-capture friendly.
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);

hipError_t launch_combine(const float* y, const int32_t* inv, const float* w, int T, int k, int H,
                          void* out, bool out_f32, hipStream_t s);

// ---- expert FFN (low-bit formats)
struct LowbitWeights {
  int fmt;  // 1 = 2-bit codebook, 2 = 3-bit
  const void* w1_codes;
  const void* w1_scales;
  const void* w2_codes;
  const void* w2_scales;
  // FP4 residual of the hot experts (2-bit layers with a residual hot set; else null):
  // MXFP4 arrays stacked along the hot slots, W1 [n_hot][2I][H/2], W2 [n_hot][H][I/2]
  const void* res_w1_codes = nullptr;
  const void* res_w1_scales = nullptr;
  const void* res_w2_codes = nullptr;
  const void* res_w2_scales = nullptr;
};

// Work list of grouped-row chunks built on the device from `offsets`.
//   int32 header[4]: [0] = number of items; then int4 items {expert, first row, rows, hot slot}.
size_t plan_bytes(int64_t max_items);
// One launch: the two low-bit work lists (streaming items of <= small_max rows; grouped-GEMM
// items of <= gemm_chunk rows for experts above small_max if gemm_enabled), and (if xp) x
// stored in the k-slot order of the weight format `fmt` (1 = 2-bit, 2 = 3-bit).  Hot experts
// are left out (they run on the FP8 path), unless hot_residual: then they join the streaming
// list whatever their size, their items carrying their hot slot.
hipError_t launch_prepare(const int32_t* offsets, int E, int small_max, int gemm_chunk, bool gemm_enabled,
                          const int32_t* hot_ids, int n_hot, bool hot_residual, int32_t* plan_s,
                          int32_t* plan_g, const uint16_t* x, int T, int H, int fmt, uint16_t* xp,
                          hipStream_t s);

// Routing, grouping and stage 0 of the FFN (front.hip) for R = T*k <= kPermuteChunk: one launch
// for T <= kFrontOneLaunchT, else the route kernel and then one launch for the rest.  nchunks and
// nbits are set by launch_front.
constexpr int kFrontOneLaunchT = 16;
struct FrontArgs {
  const float* logits;
  int T, E, k, nbits;
  int32_t *ids, *counts, *offsets, *perm, *inv;
  float* gates;
  int small_max, gemm_chunk, gemm_enabled;
  const int32_t* hot_ids;
  int n_hot, hot_residual;
  int32_t *plan_s, *plan_g;
  const uint4* x;
  int nchunks, fmt;
  uint4* xp;
};
hipError_t launch_front(const FrontArgs& a, int H, hipStream_t s);

// Decode-style kernels: weight-streaming, MFMA on 16-token tiles.
// split_T: the batch size the K split across a workgroup's waves is chosen for (T itself, or 1
// for a split that does not depend on the batch)
hipError_t launch_lowbit_fc1(const LowbitWeights& w, int E, int H, int I, int k,
                             const uint16_t* xp, const int32_t* perm, const int32_t* plan,
                             int max_items, int T, int split_T, uint16_t* hbuf, hipStream_t s);
hipError_t launch_lowbit_fc2(const LowbitWeights& w, int E, int H, int I, int k,
                             const uint16_t* hbuf, const int32_t* plan, int max_items, int T,
                             int split_T, float* y, hipStream_t s);

// Prefill-sized groups: grouped GEMM on MFMA 32x32x16 with the codes decoded into LDS tiles.
// Work items of at most kGemmRows rows.
constexpr int kGemmRows = 128;
hipError_t launch_lowbit_gemm_fc1(const LowbitWeights& w, int H, int I, int k, const uint16_t* xp,
                                  const int32_t* perm, const int32_t* plan, int max_items, int T,
                                  uint16_t* hbuf, hipStream_t s);
hipError_t launch_lowbit_gemm_fc2(const LowbitWeights& w, int H, int I, int k,
                                  const uint16_t* hbuf, const int32_t* plan, int max_items, int T,
                                  float* y, hipStream_t s);

// ---- hot experts (MXFP4 held, converted to FP8 into workspace slots, MXFP8 activations)
struct HotWeights {
  int E;  // experts of the layer (hot ids outside [0, E) are ignored)
  int n_hot;
  const int32_t* hot_ids;
  const uint8_t* w1_codes;   // [n_hot][2I][H/2]
  const uint8_t* w1_scales;  // [n_hot][2I][H/32]
  const uint8_t* w2_codes;   // [n_hot][H][I/2]
  const uint8_t* w2_scales;  // [n_hot][H][I/32]
};
// Byte layout of one workspace slot: the FP8 image of one hot expert.
struct HotLayout {
  int64_t w1_off, w1s_off, w2_off, w2s_off, slot_bytes;
};
HotLayout hot_layout(int H, int I);

hipError_t launch_mxfp8_quantize(const uint16_t* x, int64_t rows, int K, uint8_t* elems,
                                 uint8_t* scales, hipStream_t s);
hipError_t launch_mxfp4_to_fp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int K,
                               uint8_t* elems, uint8_t* out_scales, hipStream_t s);
// Quantisers (quant.hip): fp32 [rows][K] -> 2-bit codes + bf16 scales, or MXFP4.
hipError_t launch_quantize_w2(const float* w, int64_t rows, int K, uint32_t* codes, uint16_t* scales,
                              hipStream_t s);
hipError_t launch_quantize_mxfp4(const float* w, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s);
// Hot work list (items of <= chunk_rows rows of hot experts) and MXFP8 of x, in one launch.
hipError_t launch_hot_prepare(const int32_t* offsets, int E, int chunk_rows, const int32_t* hot_ids,
                              int n_hot, int32_t* plan, const uint16_t* x, int T, int H, uint8_t* xq,
                              uint8_t* xqs, hipStream_t s);
// Convert hot experts b0 .. b0+S-1 that have rows (counts > 0) into slots 0 .. S-1.
hipError_t launch_hot_convert(const HotWeights& hw, int H, int I, const int32_t* counts, int b0,
                              int S, uint8_t* slots, hipStream_t s);
// FP8 grouped GEMMs over the hot work list, for the experts in slots b0 .. b0+S-1.
hipError_t launch_hot_fc1(int H, int I, int k, int T, const int32_t* hot_plan, int max_items, int b0,
                          int S, const uint8_t* slots, const uint8_t* xq, const uint8_t* xqs,
                          const int32_t* perm, uint8_t* hq, uint8_t* hqs, hipStream_t s);
hipError_t launch_hot_fc2(int H, int I, int64_t R, const int32_t* hot_plan, int max_items, int b0,
                          int S, const uint8_t* slots, const uint8_t* hq, const uint8_t* hqs,
                          float* y, hipStream_t s);

hipError_t launch_debug_dequant(const LowbitWeights& w, int E, int H, int I, int e, int which,
                                float* out, hipStream_t s);
// The FP4 residual of hot slot `slot` through the streaming kernels' residual decoder.
hipError_t launch_debug_dequant_residual(const LowbitWeights& w, int H, int I, int slot, int which, float* out,
                                         hipStream_t s);
// The same through the grouped GEMM's field decoder (F::table32 / F::decode32).
hipError_t launch_debug_dequant_gemm(const LowbitWeights& w, int H, int I, int e, int which, float* out,
                                     hipStream_t s);

}  // namespace bitmoe
