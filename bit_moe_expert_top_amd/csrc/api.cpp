// C ABI of the low-bit MoE library (declared in include/bitmoe.h): argument checks,
// workspace layout and kernel dispatch.  No allocation, no host synchronisation.
#include <hip/hip_runtime.h>

#include "../../include/bitmoe.h"
#include "kernels.h"

using namespace bitmoe;

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxTopK = 64;

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

inline moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Rows per work item of the streaming kernels: a group of one expert is split into items
// of at most 32 rows (two 16-token MFMA tiles).
constexpr int kStreamChunk = 32;
// Batches of at least this many tokens run the grouped-GEMM kernels (prefill shape).
constexpr int kGemmMinTokens = 128;

struct FfnLayout {
  bool gemm;
  int chunk;
  int64_t max_items;
  size_t plan_off, xp_off, h_off, total;
};

FfnLayout ffn_layout(const moe_weights* w, int T, int k) {
  FfnLayout L;
  const int64_t R = (int64_t)T * k;
  L.gemm = T >= kGemmMinTokens;
  L.chunk = L.gemm ? kGemmRows : kStreamChunk;
  L.max_items = (R + L.chunk - 1) / L.chunk + (R < w->E ? R : w->E);
  size_t off = 0;
  L.plan_off = off;
  off = align256(off + plan_bytes(L.max_items));
  L.xp_off = off;  // x in k-slot order, T rows
  off = align256(off + (size_t)T * w->H * 2);
  L.h_off = off;  // h (bf16, k-slot order), R rows
  off = align256(off + (size_t)R * w->I * 2);
  L.total = off;
  return L;
}

moe_status check_weights(const moe_weights* w) {
  if (!w) return MOE_ERR_INVALID_ARG;
  if (w->E < 1 || w->E > kMaxE || w->H <= 0 || w->I <= 0) return MOE_ERR_INVALID_ARG;
  if (w->H % 256 || w->I % 256 || w->H > 16384 || w->I > 16384) return MOE_ERR_INVALID_ARG;
  if (w->fmt != MOE_FMT_W2 && w->fmt != MOE_FMT_W3) return MOE_ERR_INVALID_ARG;
  if (!w->w1_codes || !w->w1_scales || !w->w2_codes || !w->w2_scales) return MOE_ERR_INVALID_ARG;
  if (w->n_hot < 0 || w->n_hot > w->E) return MOE_ERR_INVALID_ARG;
  if (w->n_hot > 0 && (!w->hot_ids || !w->hot_w1_codes || !w->hot_w1_scales || !w->hot_w2_codes ||
                       !w->hot_w2_scales))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

LowbitWeights lowbit(const moe_weights* w) {
  LowbitWeights l;
  l.fmt = w->fmt == MOE_FMT_W2 ? 1 : 2;
  l.w1_codes = w->w1_codes;
  l.w1_scales = w->w1_scales;
  l.w2_codes = w->w2_codes;
  l.w2_scales = w->w2_scales;
  return l;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                     float* topk_w, void* stream) {
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E || k > kMaxTopK) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  return from_hip(launch_route(logits, T, E, k, topk_ids, topk_w, as_stream(stream)));
}

size_t moe_permute_ws_bytes(int32_t T, int32_t k, int32_t E) {
  if (T <= 0 || k <= 0 || E <= 0) return 0;
  return permute_ws_bytes((int64_t)T * k, E);
}

moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv, void* ws, size_t ws_bytes,
                       void* stream) {
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  const int64_t R = (int64_t)T * k;
  if (R >= ((int64_t)1 << 31)) return MOE_ERR_INVALID_ARG;
  if (R > 0 && (!topk_ids || !perm || !inv)) return MOE_ERR_INVALID_ARG;
  const size_t need = permute_ws_bytes(R, E);
  if (ws_bytes < need || (need > 0 && !ws)) return MOE_ERR_WORKSPACE;
  if (T == 0) {
    // empty batch: counts and offsets are all zero
    hipError_t e1 = launch_fill_i32(counts, E, 0, as_stream(stream));
    hipError_t e2 = launch_fill_i32(offsets, E + 1, 0, as_stream(stream));
    return (e1 == hipSuccess && e2 == hipSuccess) ? MOE_OK : MOE_ERR_HIP;
  }
  return from_hip(launch_permute(topk_ids, (int)R, E, counts, offsets, perm, inv, ws,
                                 as_stream(stream)));
}

size_t moe_expert_ffn_ws_bytes(const moe_weights* w, int32_t T, int32_t k, int32_t fp8_slots) {
  (void)fp8_slots;
  if (check_weights(w) != MOE_OK || T <= 0 || k <= 0) return 0;
  return ffn_layout(w, T, k).total;
}

namespace {

// Checks shared by moe_expert_ffn and moe_expert_ffn_stage.
moe_status ffn_check(const moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                     const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                     const float* y_perm, const void* ws, size_t ws_bytes) {
  moe_status st = check_weights(w);
  if (st != MOE_OK) return st;
  if (T < 0 || k < 1 || k > w->E) return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * k >= ((int64_t)1 << 31)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !counts || !offsets || !perm || !y_perm) return MOE_ERR_INVALID_ARG;
  if (w->n_hot != 0) return MOE_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < ffn_layout(w, T, k).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

constexpr int kFfnStages = 3;  // prepare, FC1 + SwiGLU, FC2

moe_status ffn_run_stage(const moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                         const int32_t* offsets, const int32_t* perm, float* y_perm, void* ws,
                         int stage, hipStream_t s) {
  const FfnLayout L = ffn_layout(w, T, k);
  char* base = static_cast<char*>(ws);
  int32_t* plan = reinterpret_cast<int32_t*>(base + L.plan_off);
  uint16_t* xp = reinterpret_cast<uint16_t*>(base + L.xp_off);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(base + L.h_off);
  const LowbitWeights lw = lowbit(w);
  hipError_t e = hipSuccess;
  switch (stage) {
    case 0:
      e = launch_prepare(offsets, w->E, L.chunk, w->hot_ids, w->n_hot, false, plan, x, T, w->H, lw.fmt, xp, s);
      break;
    case 1:
      e = L.gemm ? launch_lowbit_gemm_fc1(lw, w->H, w->I, k, xp, perm, plan, (int)L.max_items, T, hbuf, s)
                 : launch_lowbit_fc1(lw, w->E, w->H, w->I, k, xp, perm, plan, (int)L.max_items, T, hbuf, s);
      break;
    case 2:
      e = L.gemm ? launch_lowbit_gemm_fc2(lw, w->H, w->I, k, hbuf, plan, (int)L.max_items, T, y_perm, s)
                 : launch_lowbit_fc2(lw, w->E, w->H, w->I, k, hbuf, plan, (int)L.max_items, T, y_perm, s);
      break;
    default:
      return MOE_ERR_INVALID_ARG;
  }
  return from_hip(e);
}

}  // namespace

moe_status moe_expert_ffn(const moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                          const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                          float* y_perm, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = ffn_check(w, x, T, k, counts, offsets, perm, y_perm, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  for (int stage = 0; stage < kFfnStages && st == MOE_OK; ++stage)
    st = ffn_run_stage(w, x, T, k, offsets, perm, y_perm, ws, stage, as_stream(stream));
  return st;
}

int32_t moe_expert_ffn_num_stages(const moe_weights* w, int32_t T, int32_t k) {
  (void)w; (void)T; (void)k;
  return kFfnStages;
}

moe_status moe_expert_ffn_stage(const moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                                const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                                float* y_perm, void* ws, size_t ws_bytes, int32_t stage,
                                void* stream) {
  moe_status st = ffn_check(w, x, T, k, counts, offsets, perm, y_perm, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (stage < 0 || stage >= kFfnStages) return MOE_ERR_INVALID_ARG;
  return ffn_run_stage(w, x, T, k, offsets, perm, y_perm, ws, stage, as_stream(stream));
}

moe_status moe_combine(const float* y_perm, const int32_t* inv, const float* topk_w, int32_t T,
                       int32_t k, int32_t H, void* out, int32_t out_is_fp32, void* stream) {
  if (T < 0 || k < 1 || k > kMaxTopK * 16 || H <= 0 || H % 4) return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * k >= ((int64_t)1 << 31)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!y_perm || !inv || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  return from_hip(launch_combine(y_perm, inv, topk_w, T, k, H, out, out_is_fp32 != 0,
                                 as_stream(stream)));
}

moe_status moe_mxfp4_to_fp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t K,
                            uint8_t* elems, uint8_t* out_scales, void* stream) {
  (void)codes; (void)scales; (void)rows; (void)K; (void)elems; (void)out_scales; (void)stream;
  return MOE_ERR_UNSUPPORTED;
}

moe_status moe_mxfp8_quantize(const uint16_t* x, int64_t rows, int32_t K, uint8_t* elems,
                              uint8_t* scales, void* stream) {
  (void)x; (void)rows; (void)K; (void)elems; (void)scales; (void)stream;
  return MOE_ERR_UNSUPPORTED;
}

moe_status moe_debug_dequant(const moe_weights* w, int32_t e, int32_t which, float* out,
                             void* stream) {
  moe_status st = check_weights(w);
  if (st != MOE_OK) return st;
  if (e < 0 || e >= w->E || (which != 1 && which != 2) || !out) return MOE_ERR_INVALID_ARG;
  return from_hip(launch_debug_dequant(lowbit(w), w->E, w->H, w->I, e, which, out,
                                       as_stream(stream)));
}

}  // extern "C"
