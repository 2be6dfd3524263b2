/*
 * bitmoe.h -- C ABI of the low-bit routed-expert MoE FFN for AMD MI355X (gfx950).
 *
 * One MoE layer is four calls, in this order, all enqueued on one HIP stream:
 *
 *   moe_route      router logits            -> top-k expert ids and gates
 *   moe_permute    expert ids               -> per-expert counts/offsets, grouping perm/inv
 *   moe_expert_ffn tokens + grouped rows    -> FC1 + SwiGLU + FC2 of each row's expert
 *   moe_combine    expert outputs + gates   -> one output row per token
 *
 * Sources, by page title and section:
 *   [Moet-QA]      mhpn.cn Q&A on the vLLM-Moet project (2-bit experts on the sign-symmetric
 *                  codebook {-4,-1,1,4}; the FP4 set of hot experts).
 *   [Moet-README]  ossradar.top page "vLLM-Moet": release notes of v2026.11.03-r23 (the prefill
 *                  MoE as FC1 + SwiGLU + MXFP8 quantisation, then FC2) and the README tables
 *                  (routed experts, MXFP4 checkpoint, graph-captured decode step).
 *   [Strata-R9700] lcz.me thread on porting Strata to the R9700, path 6 (3-bit experts: eight
 *                  levels, e4m3 scale / 64, 32 codes in three 32-bit words).
 *   [Day0-MXFP4]   ruibaoantu.com article on a day-0 MoE port, section 4 (MXFP4 experts
 *                  converted online to FP8 in a reused workspace) and section 5 (the conversion
 *                  workspace kept apart from other buffers).
 *   [OCP-MX]       OCP Microscaling Formats v1.0 (e8m0, e2m1, e4m3fn, the MX scale rule).
 *
 * Conventions shared by every call:
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except `moe_weights*`
 *     itself (a host struct whose members are device pointers).  The library allocates no
 *     device memory and keeps no mutable global state; scratch lives in the caller's `ws`.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls only
 *     enqueue work and never synchronise the host, so a layer can be captured in a HIP graph.
 *   - Argument errors are detected on the host and returned before anything is enqueued.
 *     A failed launch returns MOE_ERR_HIP.  Faults inside kernels surface, as usual in HIP,
 *     at the caller's next synchronisation.
 *   - T = 0 is valid for every call and enqueues nothing.
 *   - Inputs are trusted to be finite (NaN router logits are the caller's error).
 *
 * Shapes: T tokens, E experts, k experts per token (1 <= k <= E <= 1024), H hidden size,
 * I expert intermediate size, R = T*k routed rows.  All arrays are row-major.
 */
#ifndef BITMOE_H
#define BITMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size or shape, k out of range        */
  MOE_ERR_UNSUPPORTED = -2, /* a valid request the library does not implement           */
  MOE_ERR_WORKSPACE = -3,   /* ws_bytes smaller than the matching *_ws_bytes() query    */
  MOE_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed                */
} moe_status;

/* Expert weight formats.  Every format stores the reduction dimension K contiguously:
 * W1 is [2I][H] per expert (rows [0,I) = gate projection, rows [I,2I) = up projection),
 * W2 is [H][I] per expert.  Scales group consecutive weights along K inside one row.
 *
 *  MOE_FMT_W2    [Moet-QA] 2-bit codebook: codes u32[rows][K/16], code i of a word at bits
 *                [2i, 2i+2), code c -> level {-4,-1,1,4}[c]; scales bf16 (u16 bits)
 *                [rows][K/32]; weight = level * scale.  K a multiple of 32.
 *                Precondition: scales are normal bf16 numbers with |scale| < 2^125 (then the
 *                decoded weights are exact bf16 values; a zero or subnormal scale decodes the
 *                +-4 levels within 2^-124 of the exact value).
 *  MOE_FMT_W3    [Strata-R9700] 3-bit, 8 levels: codes u32[rows][K/32*3], the three words of a
 *                group of 32 codes form one little-endian 96-bit field and code i sits at bits
 *                [3i, 3i+3); code c -> level {-8,-5,-3,-1,1,3,5,8}[c]; scales e4m3fn bytes
 *                [rows][K/64]; weight = level * e4m3(scale) / 64.  K a multiple of 64.
 *  MOE_FMT_MXFP4 [OCP-MX] e2m1 elements, codes u8[rows][K/2] (element 2i in the low nibble),
 *                e8m0 scale bytes [rows][K/32]; weight = e2m1 * 2^(scale-127).  Hot set only.
 */
typedef enum { MOE_FMT_W2 = 1, MOE_FMT_W3 = 2, MOE_FMT_MXFP4 = 3 } moe_wfmt;

/* One layer's experts.  Every expert not in the hot set uses `fmt` (W2 or W3); its arrays
 * are stacked along a leading [E] axis.  A hot expert ([Moet-QA]: the hottest experts are
 * kept at FP4 precision) is held in MXFP4 instead: its MXFP4 arrays are stacked along
 * [n_hot] in the order of `hot_ids`, and its slot in the low-bit arrays is never read. */
typedef struct {
  int32_t E, H, I;
  int32_t fmt;                 /* MOE_FMT_W2 or MOE_FMT_W3                                   */
  const void* w1_codes;        /* [E][2I][...] low-bit codes of W1                           */
  const void* w1_scales;       /* [E][2I][...] scales of W1                                  */
  const void* w2_codes;        /* [E][H][...]  codes of W2                                   */
  const void* w2_scales;       /* [E][H][...]  scales of W2                                  */
  int32_t n_hot;               /* number of experts held in MXFP4 (0 = none)                 */
  const int32_t* hot_ids;      /* device int32[n_hot], distinct expert ids (NULL if n_hot=0) */
  const void* hot_w1_codes;    /* [n_hot][2I][H/2]  u8                                       */
  const void* hot_w1_scales;   /* [n_hot][2I][H/32] u8 e8m0                                  */
  const void* hot_w2_codes;    /* [n_hot][H][I/2]   u8                                       */
  const void* hot_w2_scales;   /* [n_hot][H][I/32]  u8 e8m0                                  */
  int32_t flags;               /* MOE_FLAG_BATCH_INVARIANT | MOE_FLAG_HOT_RESIDUAL; others:
                                  INVALID_ARG                                                */
} moe_weights;

/* [Moet-README] (results table of the DeepSeek-V4.1-Flash build, quality row): a request gives
 * the same logits at any batch size.
 * With this flag moe_expert_ffn computes every grouped row with one accumulation order that
 * does not depend on T or on the other rows of the batch (the streaming kernels for every group,
 * with one K split chosen from H, I and the format alone), so a token's output has the same bits whatever
 * batch it comes in.  Without it the K split follows T and large groups of large batches run on
 * the grouped-GEMM kernels: faster, and the bits of a token may change with T (the values
 * stay within the same tolerance of the exact result).  Routing, grouping, the FP8 hot path
 * and the combine compute each token on its own in both modes. */
#define MOE_FLAG_BATCH_INVARIANT 1

/* [Moet-QA] (the FP4 delta cache: the hottest experts keep an FP4-precision correction layer
 * above their 2-bit weights) and [Moet-README] (README line "2-bit experts on vLLM v0.24.0": a
 * 2-bit codebook plus an FP4 delta cache).
 * With this flag the hot set is a residual, not a replacement: a hot expert keeps its 2-bit
 * codes and scales in the low-bit arrays (they are read), and its MXFP4 arrays (hot_w1_codes ..,
 * stacked along [n_hot] in the order of hot_ids) hold a correction added to those weights,
 * element by element, before the matmuls: W = level * scale + e2m1 * 2^(e8m0 - 127).  The sum is
 * computed with bf16 operands and fp32 accumulation like the 2-bit experts (the FFN kernels make
 * a second pass over the residual into the same sums, so it is added before SwiGLU); there is
 * no FP8 path and no FP8 workspace.  Hot experts then run on the weight-streaming kernels at
 * any batch size.  Requires fmt == MOE_FMT_W2 (else UNSUPPORTED); residual scale bytes must lie
 * in [2, 252] (every decoded value then a normal bf16).  Without a hot set the flag has no
 * effect. */
#define MOE_FLAG_HOT_RESIDUAL 2

/* moe_route -- top-k routing ([Moet-README]: each token is served by k routed experts).
 *   logits    f32[T][E]   router logits
 *   topk_ids  i32[T][k]   out: the k largest logits' expert ids, in descending logit order;
 *                         equal logits go to the lower expert id; -0.0 equals +0.0
 *   topk_w    f32[T][k]   out: gates = softmax over the k selected logits (sum to one)
 * Errors: INVALID_ARG if T < 0, E < 1, E > 1024, k < 1, k > E or k > 64, or a null pointer. */
moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k,
                     int32_t* topk_ids, float* topk_w, void* stream);

/* moe_permute -- stable grouping of the R = T*k routed rows by expert.  Plain reading: the pages
 * compute the routed experts of a step expert by expert ([Moet-README], README tables of the
 * hybrid: the routed experts of every layer, each computed where it is held) but do not describe
 * how rows are grouped; this is the plainest grouping that lets one kernel pass handle one
 * expert's rows together.
 *   topk_ids i32[T][k]    expert of row t*k+j (values in [0, E))
 *   counts   i32[E]       out: rows routed to each expert
 *   offsets  i32[E+1]     out: exclusive prefix sum of counts (offsets[E] = R)
 *   perm     i32[R]       out: grouped row r holds routed row perm[r] = t*k+j, ordered by
 *                         (expert, token, slot)
 *   inv      i32[R]       out: inv[perm[r]] = r
 *   ws       scratch of at least moe_permute_ws_bytes(T, k, E) bytes (may be NULL if that is 0)
 * The result is deterministic (no order-dependent atomics).  Rows whose id lies outside [0, E)
 * are left out: counts and offsets count the other rows only (offsets[E] is their number), perm
 * lists them first, and the inv entries of the left-out rows and the rest of perm are not
 * written.
 * Errors: INVALID_ARG (bad sizes, null output, R >= 2^31), WORKSPACE (ws too small). */
size_t moe_permute_ws_bytes(int32_t T, int32_t k, int32_t E);
moe_status moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                       int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                       void* ws, size_t ws_bytes, void* stream);

/* moe_expert_ffn -- the routed experts ([Moet-README] release notes of -r23: FC1, SwiGLU,
 * (MXFP8 quantisation for FP8 compute), FC2).  For grouped row r of expert e, with token
 * t = perm[r] / k:
 *     a = x[t] W1_e^T (fp32 accumulation), h = silu(a[:I]) * a[I:], y_perm[r] = h W2_e^T.
 * Low-bit experts dequantise their codes inside the matmul kernels (bf16 operands, fp32
 * accumulation, h rounded to bf16).  Hot MXFP4 experts are first converted to FP8 into slots
 * of the workspace ([Day0-MXFP4] section 4), then computed with MXFP8 x and h on the FP8
 * matrix cores.  Rows of experts with no tokens are not touched.
 *   x        bf16 (u16 bits) [T][H]
 *   counts, offsets, perm   as produced by moe_permute for the same topk_ids
 *   y_perm   f32[R][H]   out (row r = grouped row r)
 *   ws       workspace of at least moe_expert_ffn_ws_bytes(w, T, k, fp8_slots) bytes
 *            (fp8_slots <= 0 or > n_hot means n_hot; ignored without a hot set).  A slot holds
 *            the FP8 image of one hot expert (3 H I * 33/32 bytes); the number of slots used is
 *            the largest that fits in ws_bytes, capped at n_hot, and the hot experts are
 *            converted and computed in batches of that many (at least one slot must fit).
 *   hot_ids  must be distinct expert ids in [0, E) (not checked: device memory).
 * Shapes: H and I must be whole scale groups (multiples of 32; of 64 for W3), else INVALID_ARG.
 * The kernels are built for H % 256 == 0, I % 256 == 0 and H, I <= 16384: other valid shapes
 * return UNSUPPORTED.  fmt W2 or W3.  T * H * 2 < 2^32 (x is addressed with 32-bit byte offsets;
 * larger batches return UNSUPPORTED: split them).
 * Errors: INVALID_ARG, UNSUPPORTED (a valid format/shape the kernels are not built for), WORKSPACE. */
size_t moe_expert_ffn_ws_bytes(const moe_weights* w, int32_t T, int32_t k, int32_t fp8_slots);
moe_status moe_expert_ffn(const moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                          const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                          float* y_perm, void* ws, size_t ws_bytes, void* stream);

/* moe_expert_ffn_noalloc -- moe_expert_ffn with its workspace inside the library, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops, harnesses that
 * forbid allocation).  It allocates nothing: the workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes, one per GPU the library runs on, held until the process ends;
 * its device address is looked up once per device, on that device's first call.  Same kernels,
 * same results as moe_expert_ffn with a caller workspace of that size (with a hot set, as many
 * FP8 slots as fit, at least one).  Every call on one GPU uses that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and must be serialised by the caller.
 * Errors: as moe_expert_ffn; WORKSPACE if the batch needs more than the static workspace
 * (moe_expert_ffn_ws_bytes(w, T, k, 1) > MOE_NOALLOC_SCRATCH_BYTES); HIP if the array's device
 * address cannot be obtained. */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
moe_status moe_expert_ffn_noalloc(const moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                                  const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                                  float* y_perm, void* stream);

/* moe_expert_ffn_stage -- run one stage of moe_expert_ffn.  Calling stages 0 .. n-1, with
 * n = moe_expert_ffn_num_stages(w, T, k, ws_bytes), in order on one stream with the same
 * arguments and workspace is exactly moe_expert_ffn.  Each stage is a single kernel launch, so
 * a caller can time the kernels one by one (HIP events on `stream`) or interleave other work.
 * Stages: 0 = low-bit work lists and x in the MFMA k-slot order; 1 = low-bit FC1 + SwiGLU of
 * the groups of <= 32 rows (weight-streaming kernel); 2 = the same for larger groups (grouped
 * GEMM, batches of >= 128 tokens; launches nothing below); 3, 4 = FC2 likewise.  With a hot
 * set (n_hot > 0): 5 = hot work list and MXFP8 of x, then for each batch of S hot experts
 * (S = FP8 slots in the workspace): convert the batch's hot experts that have rows into the
 * slots, FP8 FC1 + SwiGLU + MXFP8 of h, FP8 FC2.
 * num_stages returns 0 for invalid arguments or T = 0.
 * Errors: as moe_expert_ffn; INVALID_ARG for a stage out of range. */
int32_t moe_expert_ffn_num_stages(const moe_weights* w, int32_t T, int32_t k, size_t ws_bytes);
moe_status moe_expert_ffn_stage(const moe_weights* w, const uint16_t* x, int32_t T, int32_t k,
                                const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                                float* y_perm, void* ws, size_t ws_bytes, int32_t stage,
                                void* stream);

/* moe_route_permute_prepare -- moe_route, moe_permute and stage 0 of moe_expert_ffn in one
 * launch for up to 16 tokens, in two (routing, then the rest) for up to R = T*k = 4096 rows:
 * a decode step is a chain of short kernels whose fixed start and drain costs add up, and the
 * pages capture their decode step in a graph for that reason ([Moet-README] README tables,
 * graph-captured decode).  Same arguments as those three calls
 * (topk_ids i32[T][k], topk_w f32[T][k], counts i32[E], offsets i32[E+1], perm i32[R],
 * inv i32[R], the FFN workspace ws of moe_expert_ffn_ws_bytes); the outputs and the workspace
 * contents are bit-equal to moe_route + moe_permute + moe_expert_ffn_stage(..., 0, ...), so
 * stages 1 .. n-1 of moe_expert_ffn_stage then complete the FFN.  All pointers are device
 * pointers owned by the caller; the call only enqueues on `stream`.
 * Errors: INVALID_ARG (bad weights, T < 0, k out of [1, min(E, 64)], null pointers),
 * UNSUPPORTED for T*k > 4096 (use the three calls), WORKSPACE as moe_expert_ffn.  T = 0 fills
 * counts and offsets with zeros, as moe_permute does. */
moe_status moe_route_permute_prepare(const moe_weights* w, const float* logits, const uint16_t* x,
                                     int32_t T, int32_t k, int32_t* topk_ids, float* topk_w,
                                     int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                     void* ws, size_t ws_bytes, void* stream);

/* moe_expert_ffn_ws_region -- where an intermediate result of moe_expert_ffn lives in its
 * workspace, so that a test can read it back after the stage that writes it (the pages check a
 * conversion by comparing its output on fixed inputs: [Day0-MXFP4] section 4, the consistency
 * check after the online conversion).  For the same (w, T, k, ws_bytes) as the FFN call:
 *   MOE_WS_XQ          u8[T][H]     MXFP8 elements of x (stage 5, hot set only)
 *   MOE_WS_XQ_SCALES   u8[T][H/32]  their e8m0 scales
 *   MOE_WS_HQ          u8[R][I]     MXFP8 h of the rows of hot experts (row r = grouped row r,
 *                                   columns in natural order), written by the FP8 FC1 stage of
 *                                   the batch that holds the row's expert; other rows untouched
 *   MOE_WS_HQ_SCALES   u8[R][I/32]  their e8m0 scales
 *   MOE_WS_SLOTS       the S FP8 slots, S * slot_bytes (see moe_fp8_slot_layout): slot j holds
 *                      the converted image of hot expert b0 + j of the current batch, written by
 *                      that batch's convert stage only if the expert has rows
 * *offset and *bytes receive the region's byte offset in ws and its size.
 * Errors: INVALID_ARG (bad weights or sizes, unknown region, null outputs), UNSUPPORTED (a hot
 * region without a hot set), WORKSPACE (ws_bytes too small for the call). */
typedef enum {
  MOE_WS_XQ = 1,
  MOE_WS_XQ_SCALES = 2,
  MOE_WS_HQ = 3,
  MOE_WS_HQ_SCALES = 4,
  MOE_WS_SLOTS = 5
} moe_ws_region;
moe_status moe_expert_ffn_ws_region(const moe_weights* w, int32_t T, int32_t k, size_t ws_bytes,
                                    int32_t region, size_t* offset, size_t* bytes);

/* moe_fp8_slot_layout -- byte layout of one FP8 slot ([Day0-MXFP4] section 4: the converted
 * image of one MXFP4 expert): W1 e4m3fn elements u8[2I][H] at *w1, their e8m0 scales
 * u8[2I][H/32] at *w1_scales, W2 elements u8[H][I] at *w2, scales u8[H][I/32] at *w2_scales
 * (offsets from the slot's start), and the slot size (the stride between slots).
 * Errors: INVALID_ARG (H or I not positive multiples of 32, null outputs). */
moe_status moe_fp8_slot_layout(int32_t H, int32_t I, size_t* w1, size_t* w1_scales, size_t* w2,
                               size_t* w2_scales, size_t* slot_bytes);

/* moe_combine -- out[t] = sum over j = 0..k-1 (in that order) of topk_w[t][j] * y_perm[inv[t*k+j]],
 * accumulated in fp32.  Plain reading: the pages do not describe the combine; this is the
 * gate-weighted sum of a token's routed-expert outputs that the gates of moe_route define.  out is f32[T][H] if out_is_fp32, else bf16 (u16 bits, round to
 * nearest even of the same fp32 sum).
 * Errors: INVALID_ARG. */
moe_status moe_combine(const float* y_perm, const int32_t* inv, const float* topk_w,
                       int32_t T, int32_t k, int32_t H, void* out, int32_t out_is_fp32,
                       void* stream);

/* moe_mxfp4_to_fp8 -- [Day0-MXFP4] section 4: convert an MXFP4 matrix to FP8.  Each e2m1
 * element becomes the e4m3fn byte of the same value (lossless, -0 -> 0x80); e8m0 scales are
 * copied.  This is the conversion moe_expert_ffn runs on hot experts.
 *   codes u8[rows][K/2], scales u8[rows][K/32] -> elems u8[rows][K], out_scales u8[rows][K/32]
 * Errors: INVALID_ARG (K % 32 != 0, null pointer). */
moe_status moe_mxfp4_to_fp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t K,
                            uint8_t* elems, uint8_t* out_scales, void* stream);

/* moe_mxfp8_quantize -- [OCP-MX] MXFP8 (e4m3fn) quantisation of bf16 rows, blocks of 32 along K:
 * shared exponent floor(log2(amax)) - 8 (scale byte 0 for an all-zero block), elements
 * round-to-nearest-even and saturate at +-448.  The quantisation moe_expert_ffn applies to
 * the FC1 input of hot experts.
 *   x bf16 [rows][K] -> elems u8[rows][K], scales u8[rows][K/32].   Errors: INVALID_ARG. */
moe_status moe_mxfp8_quantize(const uint16_t* x, int64_t rows, int32_t K, uint8_t* elems,
                              uint8_t* scales, void* stream);

/* moe_quantize_w2 -- fit fp32 weights to the 2-bit codebook format ([Moet-QA]: 2-bit experts on
 * the codebook {-4,-1,1,4}; the pages do not give the fitting procedure).  Per group of 32
 * consecutive weights along K of one row: the least-squares fit w ~ level[code] * s by
 * alternating nearest-level codes and the scale sum(level*w)/sum(level^2), from
 * s = max|w|/4, three rounds, then s rounded to bf16 (nearest even) and the final codes
 * chosen against that stored scale.  All decisions in fp32 in a fixed order (deterministic);
 * nearest-level rule with t = 2.5 s: +4 if w > t, +1 if 0 <= w <= t, -1 if -t <= w < 0,
 * -4 if w < -t.  An all-zero group gets scale 0 and code 2 (+1).
 *   w f32[rows][K] (finite) -> codes u32[rows][K/16] (code i of a word at bits [2i, 2i+2)),
 *   scales u16[rows][K/32] (bf16 bits).  The output is the MOE_FMT_W2_CB4_G32_BF16 layout of
 *   one weight matrix (W1 of an expert is [2I][H], W2 is [H][I]).
 * Errors: INVALID_ARG (rows < 0, K not a positive multiple of 32, null pointer with rows > 0). */
moe_status moe_quantize_w2(const float* w, int64_t rows, int32_t K, uint32_t* codes, uint16_t* scales,
                           void* stream);

/* moe_quantize_mxfp4 -- [OCP-MX] MXFP4 quantisation of fp32 weights, blocks of 32 along K:
 * shared exponent floor(log2(amax)) - 2, clamped to [-127, 127] (scale byte 0 for an all-zero
 * block); elements w / 2^shared rounded to the nearest e2m1 value, ties to the even mantissa,
 * saturating at +-6; the sign of -0 is kept.
 *   w f32[rows][K] (finite) -> codes u8[rows][K/2] (element 2i in the low nibble),
 *   scales u8[rows][K/32] (e8m0) -- the MOE_FMT_MXFP4 layout.
 * Errors: INVALID_ARG as moe_quantize_w2. */
moe_status moe_quantize_mxfp4(const float* w, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                              void* stream);

/* ---------------------------------------------------------------- host-RAM expert tier
 * [Moet-QA] (section on what the project teaches): when the experts outgrow the GPU, most of
 * them stay in host RAM and the GPU serves as a cache of the hot ones, which routing locality
 * makes hit most of the work.  [Moet-README] (flagship results; launcher): the cache is an LRU
 * over a budget of expert slots.  Reading: every expert a batch routes to is made resident
 * before the batch runs (misses are copied host -> device, not computed elsewhere); a miss takes
 * the lowest empty slot, else the least recently used slot that this batch does not use.
 *
 * Use: route the batch; copy its topk_ids to the host; moe_tier_plan; moe_tier_load the
 * planned experts; copy slot_of_expert to the device; moe_tier_remap the ids to slot ids; run
 * moe_permute / moe_expert_ffn / moe_combine with E = n_slots on the slot arrays (a
 * moe_weights whose E is n_slots and whose arrays hold n_slots experts).  The per-row
 * arithmetic is the same as with every expert resident, so the output is bit for bit the same.
 * The tier holds low-bit experts only (no MXFP4 hot set). */
typedef struct {
  int32_t E;                /* experts of the layer                                          */
  int32_t n_slots;          /* experts the GPU holds                                         */
  int32_t* slot_of_expert;  /* host int32[E]: slot of a resident expert, -1 if not resident  */
  int32_t* expert_of_slot;  /* host int32[n_slots]: expert in a slot, -1 if the slot is empty */
  int64_t* last_use;        /* host int64[n_slots]: tick of the last batch that used the slot */
  int64_t tick;             /* batches planned so far (0 for a fresh state, all slots empty) */
} moe_tier_state;

/* moe_tier_plan -- host only, no device call.  Marks the experts that ids[0..R) route to as used
 * by the next batch (tick + 1), keeps the resident ones in place and assigns each missing one a
 * slot, in ascending expert id order: the lowest empty slot, else the slot with the smallest
 * last_use among the slots this batch does not use (ties: lowest slot).  Updates the state and
 * writes the n_load experts to copy and their slots to load_expert / load_slot (host, room for
 * n_slots entries each).
 * Errors: INVALID_ARG (null pointer, id outside [0, E), bad sizes); UNSUPPORTED if the batch
 * routes to more distinct experts than n_slots (the state is left unchanged: split the batch). */
moe_status moe_tier_plan(moe_tier_state* st, const int32_t* ids, int64_t R, int32_t* load_expert,
                         int32_t* load_slot, int32_t* n_load);

/* moe_tier_load -- enqueue on `stream` the host -> device copies of the planned experts: expert
 * load_expert[i] of host_w (E experts, arrays in host memory) into slot load_slot[i] of slot_w
 * (n_slots experts as its E, arrays in device memory), all four arrays.  Both describe the same
 * format (W2 or W3), H and I.  The host arrays should be pinned (hipHostMalloc) for the copies
 * to be asynchronous; ownership stays with the caller.  load_expert / load_slot are host arrays.
 * Errors: INVALID_ARG (format or shape mismatch, index out of range, null pointer); HIP. */
moe_status moe_tier_load(const moe_weights* host_w, const moe_weights* slot_w, const int32_t* load_expert,
                         const int32_t* load_slot, int32_t n_load, void* stream);

/* moe_tier_remap -- slot_ids[i] = slot_of_expert[topk_ids[i]] for i < R, on the device (both
 * tables in device memory).  Every id must be resident (moe_tier_plan makes it so); ids are not
 * range-checked (device memory).
 * Errors: INVALID_ARG (R < 0, null pointer with R > 0); HIP. */
moe_status moe_tier_remap(const int32_t* topk_ids, int64_t R, const int32_t* slot_of_expert,
                          int32_t* slot_ids, void* stream);

/* moe_debug_dequant -- decode one low-bit expert matrix with the same device code the FFN
 * kernels use, into f32[rows][K] (W1: rows = 2I, K = H; W2: rows = H, K = I), in natural K
 * order.  For tests: the decoded weights must equal the format definition bit for bit.
 *   which: 1 (W1) or 2 (W2) through the weight-streaming kernels' decoder; 3 (W1) or 4 (W2)
 *          through the grouped-GEMM kernels' decoder (one 32-k field per lane); 5 (W1) or 6
 *          (W2): the FP4 residual of hot slot e (MOE_FLAG_HOT_RESIDUAL layers only, else
 *          UNSUPPORTED) through the streaming kernels' residual decoder.
 * Errors: INVALID_ARG, UNSUPPORTED. */
moe_status moe_debug_dequant(const moe_weights* w, int32_t e, int32_t which, float* out,
                             void* stream);

/* Human-readable name of a status code (static string). */
const char* moe_status_str(moe_status s);

#ifdef __cplusplus
}
#endif
#endif /* BITMOE_H */
