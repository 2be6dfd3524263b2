// C ABI of the low-bit MoE library (declared in include/bitmoe.h): argument checks,
// workspace layout and kernel dispatch.  No allocation, no host synchronisation.
#include <hip/hip_runtime.h>

#include <mutex>

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
// of at most 32 rows (two 16-token MFMA tiles); in batches of <= 16 tokens at most 16 rows:
// there the streaming kernel splits K across its waves and its token stage holds one 16-row
// tile per K part.  (With distinct experts per token a group never exceeds T rows; repeated
// ids can make it larger.)
constexpr int kStreamChunk = 32;
// In batches of at least this many tokens, the groups larger than kStreamChunk rows run on the
// grouped-GEMM kernels (items of kGemmRows rows); smaller groups always stream.
constexpr int kGemmMinTokens = 128;

// Batch-invariant mode: every group streams, and the streaming kernels take the K split of a
// 16-token batch whatever T is (it then depends on H, I and the format only).  A row's sums are
// formed in the same order for every T: the split fixes how K is cut and summed, and the kernels
// treat each token column of a tile on its own, so the item size (16 or 32 rows) does not matter.
inline bool invariant(const moe_weights* w) { return (w->flags & MOE_FLAG_BATCH_INVARIANT) != 0; }
// A hot set held as an FP4 residual on top of the experts' 2-bit codes: no FP8 path, the hot
// experts stream with a second (residual) pass.
inline bool hot_residual(const moe_weights* w) { return (w->flags & MOE_FLAG_HOT_RESIDUAL) != 0 && w->n_hot > 0; }
// A hot set computed on the FP8 path (MXFP4 held, converted into workspace slots).
inline bool hot_fp8(const moe_weights* w) { return w->n_hot > 0 && !hot_residual(w); }
inline int stream_chunk(int T) { return T <= 16 ? 16 : kStreamChunk; }
inline int split_tokens(const moe_weights* w, int T) { return invariant(w) ? 16 : T; }

// Hot experts are computed by the FP8 grouped GEMM on items of this many rows.
constexpr int kHotChunk = 128;

struct FfnLayout {
  bool gemm;                    // the grouped-GEMM list is in use
  int64_t max_items_s, max_items_g;
  size_t plan_s_off, plan_g_off, xp_off, h_off;
  // hot experts (n_hot > 0)
  int64_t hot_max_items;
  size_t hot_plan_off, xq_off, xqs_off, hq_off, hqs_off, slots_off;
  size_t slot_bytes;
  size_t fixed;  // bytes before the FP8 slots
};

FfnLayout ffn_layout(const moe_weights* w, int T, int k) {
  FfnLayout L;
  const int64_t R = (int64_t)T * k;
  L.gemm = T >= kGemmMinTokens && !invariant(w);
  const int64_t per_expert = R < w->E ? R : w->E;  // one partial item per expert at most
  const int chunk = stream_chunk(T);
  L.max_items_s = (R + chunk - 1) / chunk + per_expert;
  L.max_items_g = L.gemm ? (R + kGemmRows - 1) / kGemmRows + per_expert : 0;
  size_t off = 0;
  L.plan_s_off = off;
  off = align256(off + plan_bytes(L.max_items_s));
  L.plan_g_off = off;
  off = align256(off + plan_bytes(L.max_items_g));
  L.xp_off = off;  // x in k-slot order, T rows
  off = align256(off + (size_t)T * w->H * 2);
  L.h_off = off;  // h (bf16, k-slot order), R rows
  off = align256(off + (size_t)R * w->I * 2);
  L.hot_max_items = 0;
  L.hot_plan_off = L.xq_off = L.xqs_off = L.hq_off = L.hqs_off = L.slots_off = off;
  L.slot_bytes = 0;
  if (hot_fp8(w)) {
    L.hot_max_items = (R + kHotChunk - 1) / kHotChunk + (R < w->n_hot ? R : w->n_hot);
    L.hot_plan_off = off;
    off = align256(off + plan_bytes(L.hot_max_items));
    L.xq_off = off;  // MXFP8 x: elements T x H, scales T x H/32
    off = align256(off + (size_t)T * w->H);
    L.xqs_off = off;
    off = align256(off + (size_t)T * (w->H / 32));
    L.hq_off = off;  // MXFP8 h of hot rows: R x I, scales R x I/32
    off = align256(off + (size_t)R * w->I);
    L.hqs_off = off;
    off = align256(off + (size_t)R * (w->I / 32));
    L.slots_off = off;
    L.slot_bytes = (size_t)hot_layout(w->H, w->I).slot_bytes;
  }
  L.fixed = off;
  return L;
}

// FP8 slots that fit in ws_bytes (capped at n_hot); 0 if none fits or there is no hot set.
int ffn_slots(const moe_weights* w, const FfnLayout& L, size_t ws_bytes) {
  if (!hot_fp8(w) || ws_bytes < L.fixed) return 0;
  const size_t s = (ws_bytes - L.fixed) / L.slot_bytes;
  return (int)(s < (size_t)w->n_hot ? s : (size_t)w->n_hot);
}

moe_status check_weights(const moe_weights* w) {
  if (!w) return MOE_ERR_INVALID_ARG;
  if (w->E < 1 || w->E > kMaxE || w->H <= 0 || w->I <= 0) return MOE_ERR_INVALID_ARG;
  if (w->fmt != MOE_FMT_W2 && w->fmt != MOE_FMT_W3) return MOE_ERR_INVALID_ARG;
  // a shape the formats define: whole scale groups along K (32 weights, 64 for 3-bit)
  const int group = w->fmt == MOE_FMT_W3 ? 64 : 32;
  if (w->H % group || w->I % group) return MOE_ERR_INVALID_ARG;
  // shapes the kernels are built for: whole 256-k steps, at most 16384
  if (w->H % 256 || w->I % 256 || w->H > 16384 || w->I > 16384) return MOE_ERR_UNSUPPORTED;
  if (!w->w1_codes || !w->w1_scales || !w->w2_codes || !w->w2_scales) return MOE_ERR_INVALID_ARG;
  if (w->n_hot < 0 || w->n_hot > w->E) return MOE_ERR_INVALID_ARG;
  if (w->flags & ~(MOE_FLAG_BATCH_INVARIANT | MOE_FLAG_HOT_RESIDUAL)) return MOE_ERR_INVALID_ARG;
  if (w->n_hot > 0 && (!w->hot_ids || !w->hot_w1_codes || !w->hot_w1_scales || !w->hot_w2_codes ||
                       !w->hot_w2_scales))
    return MOE_ERR_INVALID_ARG;
  // the FP4 residual sits on 2-bit experts
  if (hot_residual(w) && w->fmt != MOE_FMT_W2) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

HotWeights hot(const moe_weights* w) {
  HotWeights h;
  h.E = w->E;
  h.n_hot = w->n_hot;
  h.hot_ids = w->hot_ids;
  h.w1_codes = static_cast<const uint8_t*>(w->hot_w1_codes);
  h.w1_scales = static_cast<const uint8_t*>(w->hot_w1_scales);
  h.w2_codes = static_cast<const uint8_t*>(w->hot_w2_codes);
  h.w2_scales = static_cast<const uint8_t*>(w->hot_w2_scales);
  return h;
}

LowbitWeights lowbit(const moe_weights* w) {
  LowbitWeights l;
  l.fmt = w->fmt == MOE_FMT_W2 ? 1 : 2;
  l.w1_codes = w->w1_codes;
  l.w1_scales = w->w1_scales;
  l.w2_codes = w->w2_codes;
  l.w2_scales = w->w2_scales;
  if (hot_residual(w)) {
    l.res_w1_codes = w->hot_w1_codes;
    l.res_w1_scales = w->hot_w1_scales;
    l.res_w2_codes = w->hot_w2_codes;
    l.res_w2_scales = w->hot_w2_scales;
  }
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
  if (check_weights(w) != MOE_OK || T <= 0 || k <= 0) return 0;
  const FfnLayout L = ffn_layout(w, T, k);
  if (!hot_fp8(w)) return L.fixed;
  const int s = (fp8_slots <= 0 || fp8_slots > w->n_hot) ? w->n_hot : fp8_slots;
  return L.fixed + (size_t)s * L.slot_bytes;
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
  // the kernels address x (T x H bf16) and one item's rows of h with 32-bit byte offsets
  if ((int64_t)T * w->H * 2 >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  const FfnLayout L = ffn_layout(w, T, k);
  if (!ws || ws_bytes < L.fixed) return MOE_ERR_WORKSPACE;
  if (hot_fp8(w) && ffn_slots(w, L, ws_bytes) < 1) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// Stages: 0 prepare (low-bit work lists, x in k-slot order), 1 low-bit FC1 + SwiGLU on the
// streaming list, 2 the same on the grouped-GEMM list, 3 low-bit FC2 streaming, 4 FC2 grouped
// GEMM (stages 2 and 4 launch nothing below kGemmMinTokens tokens); with a hot set, 5 hot
// prepare (hot work list, MXFP8 of x), then per batch of S hot experts: convert into the
// slots, FP8 FC1 + SwiGLU + MXFP8 of h, FP8 FC2.
constexpr int kLowbitStages = 5;

int ffn_num_stages(const moe_weights* w, int T, int k, size_t ws_bytes) {
  if (!hot_fp8(w)) return kLowbitStages;
  const int S = ffn_slots(w, ffn_layout(w, T, k), ws_bytes);
  if (S < 1) return kLowbitStages + 1;
  return kLowbitStages + 1 + 3 * ((w->n_hot + S - 1) / S);
}

moe_status ffn_run_stage(const moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                         const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                         float* y_perm, void* ws, size_t ws_bytes, int stage, hipStream_t s) {
  const FfnLayout L = ffn_layout(w, T, k);
  char* base = static_cast<char*>(ws);
  int32_t* plan_s = reinterpret_cast<int32_t*>(base + L.plan_s_off);
  int32_t* plan_g = reinterpret_cast<int32_t*>(base + L.plan_g_off);
  uint16_t* xp = reinterpret_cast<uint16_t*>(base + L.xp_off);
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(base + L.h_off);
  const LowbitWeights lw = lowbit(w);
  hipError_t e = hipSuccess;
  switch (stage) {
    case 0:
      e = launch_prepare(offsets, w->E, stream_chunk(T), kGemmRows, L.gemm, w->hot_ids, w->n_hot, hot_residual(w),
                         plan_s, plan_g, x, T, w->H, lw.fmt, xp, s);
      break;
    case 1:
      e = launch_lowbit_fc1(lw, w->E, w->H, w->I, k, xp, perm, plan_s, (int)L.max_items_s, T,
                            split_tokens(w, T), hbuf, s);
      break;
    case 2:
      if (L.gemm) e = launch_lowbit_gemm_fc1(lw, w->H, w->I, k, xp, perm, plan_g, (int)L.max_items_g, T, hbuf, s);
      break;
    case 3:
      e = launch_lowbit_fc2(lw, w->E, w->H, w->I, k, hbuf, plan_s, (int)L.max_items_s, T,
                            split_tokens(w, T), y_perm, s);
      break;
    case 4:
      if (L.gemm) e = launch_lowbit_gemm_fc2(lw, w->H, w->I, k, hbuf, plan_g, (int)L.max_items_g, T, y_perm, s);
      break;
    case 5:
      e = launch_hot_prepare(offsets, w->E, kHotChunk, w->hot_ids, w->n_hot,
                             reinterpret_cast<int32_t*>(base + L.hot_plan_off), x, T, w->H,
                             reinterpret_cast<uint8_t*>(base + L.xq_off),
                             reinterpret_cast<uint8_t*>(base + L.xqs_off), s);
      break;
    default: {
      const int S = ffn_slots(w, L, ws_bytes);
      const int b0 = ((stage - kLowbitStages - 1) / 3) * S, part = (stage - kLowbitStages - 1) % 3;
      const int32_t* hplan = reinterpret_cast<const int32_t*>(base + L.hot_plan_off);
      uint8_t* slots = reinterpret_cast<uint8_t*>(base + L.slots_off);
      uint8_t* hq = reinterpret_cast<uint8_t*>(base + L.hq_off);
      uint8_t* hqs = reinterpret_cast<uint8_t*>(base + L.hqs_off);
      if (part == 0)
        e = launch_hot_convert(hot(w), w->H, w->I, counts, b0, S, slots, s);
      else if (part == 1)
        e = launch_hot_fc1(w->H, w->I, k, T, hplan, (int)L.hot_max_items, b0, S, slots,
                           reinterpret_cast<const uint8_t*>(base + L.xq_off),
                           reinterpret_cast<const uint8_t*>(base + L.xqs_off), perm, hq, hqs, s);
      else
        e = launch_hot_fc2(w->H, w->I, (int64_t)T * k, hplan, (int)L.hot_max_items, b0, S, slots, hq, hqs,
                           y_perm, s);
    }
  }
  return from_hip(e);
}

}  // namespace

moe_status moe_expert_ffn(const moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                          const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                          float* y_perm, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = ffn_check(w, x, T, k, counts, offsets, perm, y_perm, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  const int n = ffn_num_stages(w, T, k, ws_bytes);
  for (int stage = 0; stage < n && st == MOE_OK; ++stage)
    st = ffn_run_stage(w, x, T, k, counts, offsets, perm, y_perm, ws, ws_bytes, stage, as_stream(stream));
  return st;
}

int32_t moe_expert_ffn_num_stages(const moe_weights* w, int32_t T, int32_t k, size_t ws_bytes) {
  if (check_weights(w) != MOE_OK || T < 0 || k < 1) return 0;
  if (T == 0) return 0;
  return ffn_num_stages(w, T, k, ws_bytes);
}

}  // extern "C"

// ------------------------------------------------------------------ the allocation-free variant
// A workspace that lives in the library: one copy per GPU, held until the process ends.  The
// host-side name `scratch` is not a device address; its address on each device comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that address is
// passed to the kernels.
namespace {

constexpr size_t kStaticScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch array (nullptr on failure).
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

moe_status moe_expert_ffn_noalloc(const moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                                  const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                                  float* y_perm, void* stream) {
  moe_status st = check_weights(w);
  if (st != MOE_OK) return st;
  if (T < 0 || k < 1 || k > w->E || (int64_t)T * k >= ((int64_t)1 << 31)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  // the batch must fit the static workspace (with at least one FP8 slot for a hot set)
  const FfnLayout L = ffn_layout(w, T, k);
  if (L.fixed > kStaticScratchBytes || (hot_fp8(w) && ffn_slots(w, L, kStaticScratchBytes) < 1))
    return MOE_ERR_WORKSPACE;
  void* ws = device_scratch();
  if (!ws) return MOE_ERR_HIP;
  return moe_expert_ffn(w, x, T, k, counts, offsets, perm, y_perm, ws, kStaticScratchBytes, stream);
}

moe_status moe_expert_ffn_stage(const moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                                const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                                float* y_perm, void* ws, size_t ws_bytes, int32_t stage,
                                void* stream) {
  moe_status st = ffn_check(w, x, T, k, counts, offsets, perm, y_perm, ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (stage < 0 || stage >= ffn_num_stages(w, T, k, ws_bytes)) return MOE_ERR_INVALID_ARG;
  return ffn_run_stage(w, x, T, k, counts, offsets, perm, y_perm, ws, ws_bytes, stage, as_stream(stream));
}

moe_status moe_route_permute_prepare(const moe_weights* w, const float* logits, const uint16_t* x,
                                     int32_t T, int32_t k, int32_t* topk_ids, float* topk_w,
                                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                     void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_weights(w);
  if (st != MOE_OK) return st;
  if (T < 0 || k < 1 || k > w->E || k > kMaxTopK) return MOE_ERR_INVALID_ARG;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * k > kPermuteChunk) return MOE_ERR_UNSUPPORTED;  // one workgroup groups the rows
  hipStream_t s = as_stream(stream);
  if (T == 0) {  // as moe_permute: counts and offsets all zero; nothing else to do
    hipError_t e1 = launch_fill_i32(counts, w->E, 0, s);
    hipError_t e2 = launch_fill_i32(offsets, w->E + 1, 0, s);
    return (e1 == hipSuccess && e2 == hipSuccess) ? MOE_OK : MOE_ERR_HIP;
  }
  if (!logits || !x || !topk_ids || !topk_w || !perm || !inv) return MOE_ERR_INVALID_ARG;
  const FfnLayout L = ffn_layout(w, T, k);
  if (!ws || ws_bytes < L.fixed) return MOE_ERR_WORKSPACE;
  if (hot_fp8(w) && ffn_slots(w, L, ws_bytes) < 1) return MOE_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  FrontArgs a{};
  a.logits = logits;
  a.T = T;
  a.E = w->E;
  a.k = k;
  a.ids = topk_ids;
  a.gates = topk_w;
  a.counts = counts;
  a.offsets = offsets;
  a.perm = perm;
  a.inv = inv;
  a.small_max = stream_chunk(T);
  a.gemm_chunk = kGemmRows;
  a.gemm_enabled = L.gemm ? 1 : 0;
  a.hot_ids = w->hot_ids;
  a.n_hot = w->n_hot;
  a.hot_residual = hot_residual(w) ? 1 : 0;
  a.plan_s = reinterpret_cast<int32_t*>(base + L.plan_s_off);
  a.plan_g = reinterpret_cast<int32_t*>(base + L.plan_g_off);
  a.x = reinterpret_cast<const uint4*>(x);
  a.fmt = lowbit(w).fmt;
  a.xp = reinterpret_cast<uint4*>(base + L.xp_off);
  return from_hip(launch_front(a, w->H, s));
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
  if (rows < 0 || K <= 0 || K % 32) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!codes || !scales || !elems || !out_scales) return MOE_ERR_INVALID_ARG;
  return from_hip(launch_mxfp4_to_fp8(codes, scales, rows, K, elems, out_scales, as_stream(stream)));
}

moe_status moe_mxfp8_quantize(const uint16_t* x, int64_t rows, int32_t K, uint8_t* elems,
                              uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!x || !elems || !scales) return MOE_ERR_INVALID_ARG;
  return from_hip(launch_mxfp8_quantize(x, rows, K, elems, scales, as_stream(stream)));
}

moe_status moe_quantize_w2(const float* w, int64_t rows, int32_t K, uint32_t* codes, uint16_t* scales,
                           void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!w || !codes || !scales) return MOE_ERR_INVALID_ARG;
  return from_hip(launch_quantize_w2(w, rows, K, codes, scales, as_stream(stream)));
}

moe_status moe_quantize_mxfp4(const float* w, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                              void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!w || !codes || !scales) return MOE_ERR_INVALID_ARG;
  return from_hip(launch_quantize_mxfp4(w, rows, K, codes, scales, as_stream(stream)));
}

moe_status moe_debug_dequant(const moe_weights* w, int32_t e, int32_t which, float* out,
                             void* stream) {
  moe_status st = check_weights(w);
  if (st != MOE_OK) return st;
  if (e < 0 || e >= w->E || which < 1 || which > 6 || !out) return MOE_ERR_INVALID_ARG;
  if (which >= 5) {  // the FP4 residual of hot slot e
    if (!hot_residual(w)) return MOE_ERR_UNSUPPORTED;
    if (e >= w->n_hot) return MOE_ERR_INVALID_ARG;
    return from_hip(launch_debug_dequant_residual(lowbit(w), w->H, w->I, e, which - 4, out, as_stream(stream)));
  }
  if (which <= 2)
    return from_hip(launch_debug_dequant(lowbit(w), w->E, w->H, w->I, e, which, out, as_stream(stream)));
  return from_hip(launch_debug_dequant_gemm(lowbit(w), w->H, w->I, e, which - 2, out, as_stream(stream)));
}

moe_status moe_expert_ffn_ws_region(const moe_weights* w, int32_t T, int32_t k, size_t ws_bytes,
                                    int32_t region, size_t* offset, size_t* bytes) {
  moe_status st = check_weights(w);
  if (st != MOE_OK) return st;
  if (T < 1 || k < 1 || k > w->E || (int64_t)T * k >= ((int64_t)1 << 31) || !offset || !bytes)
    return MOE_ERR_INVALID_ARG;
  if (region < MOE_WS_XQ || region > MOE_WS_SLOTS) return MOE_ERR_INVALID_ARG;
  if (!hot_fp8(w)) return MOE_ERR_UNSUPPORTED;
  const FfnLayout L = ffn_layout(w, T, k);
  const int S = ffn_slots(w, L, ws_bytes);
  if (S < 1) return MOE_ERR_WORKSPACE;
  const size_t R = (size_t)T * k;
  switch (region) {
    case MOE_WS_XQ: *offset = L.xq_off; *bytes = (size_t)T * w->H; break;
    case MOE_WS_XQ_SCALES: *offset = L.xqs_off; *bytes = (size_t)T * (w->H / 32); break;
    case MOE_WS_HQ: *offset = L.hq_off; *bytes = R * w->I; break;
    case MOE_WS_HQ_SCALES: *offset = L.hqs_off; *bytes = R * (w->I / 32); break;
    default: *offset = L.slots_off; *bytes = (size_t)S * L.slot_bytes; break;
  }
  return MOE_OK;
}

moe_status moe_fp8_slot_layout(int32_t H, int32_t I, size_t* w1, size_t* w1_scales, size_t* w2,
                               size_t* w2_scales, size_t* slot_bytes) {
  if (H < 32 || I < 32 || H % 32 || I % 32 || !w1 || !w1_scales || !w2 || !w2_scales || !slot_bytes)
    return MOE_ERR_INVALID_ARG;
  const HotLayout L = hot_layout(H, I);
  *w1 = (size_t)L.w1_off;
  *w1_scales = (size_t)L.w1s_off;
  *w2 = (size_t)L.w2_off;
  *w2_scales = (size_t)L.w2s_off;
  *slot_bytes = (size_t)L.slot_bytes;
  return MOE_OK;
}

}  // extern "C"
