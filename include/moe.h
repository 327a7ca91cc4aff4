/*
 * moe.h — C ABI of a dropless mixture-of-experts layer (forward and backward) for AMD
 * Instinct MI355X (gfx950).  Library: libmoe.so.
 *
 * Pages the operations are defined on (titles as published; headings translated in []):
 *   [Prime] "Prime Mega MoE: tanításra is jó a DeepSeek MoE kernele" (neuraldaily.news)
 *   [JAX]   "Az NVIDIA szerint tízszer gyorsabb lett a dropless MoE tanítása JAX-ban" (aihirek.info)
 *   [TE]    "NVIDIA מציגה דרך יעילה לאמן מודלי MoE בביולוגיה" (sitech.ge)
 *   [Mega]  the DeepGEMM "Mega MoE" announcement on itsolotime.com
 *
 * Notation: T tokens, d model dim, f expert FFN dim, E experts, k slots per token.  A pair
 * p = t*k + j is slot j of token t.  A = T*k is the maximum number of routed pairs; buffers are
 * sized by it, never by E x capacity (dropless: [JAX] "A dropless MoE minden tokent
 * feldolgoz" [dropless MoE processes every token]).
 *
 * Layouts (all row-major, contiguous, device memory unless stated):
 *   x, dx, y, dy   bf16 [T, d]              (fp8: x is e4m3 [T, d] with x_scale fp32 [T, d/128])
 *   W1, dW1        bf16 [E, d, 2f]          columns [0,f) are the gate, [f,2f) the up projection
 *                                           (fp8: e4m3 with W1_scale fp32 [E, d/128, 2f/128])
 *   W2, dW2        bf16 [E, f, d]           (fp8: e4m3 with W2_scale fp32 [E, f/128, d/128])
 *   logits, d_logits  fp32 [T, E]
 *   topk_ids       int32 [T, k]  slot j = j-th largest logit, ties to the lower id; -1 = the
 *                                slot is not routed here (pre-routed input only)
 *   topk_w, d_topk_w  fp32 [T, k]
 *   counts         int32 [E]     routed pairs per expert
 *   offsets        int32 [E+1]   exclusive prefix sum of counts; offsets[E] = routed pairs
 *   perm           int32 [T*k]   sorted position -> pair p (entries >= offsets[E] unused)
 *   inv_perm       int32 [T*k]   pair p -> sorted position, -1 for a slot that is not routed
 * The sorted order is expert-major, then ascending pair index within an expert (a stable
 * counting sort), which makes it unique and bit-reproducible.
 *
 * Conventions for every call:
 *   - Ownership: the caller allocates every buffer (including `ws` workspace and the `saved`
 *     forward->backward context).  The library allocates nothing and keeps no state between
 *     calls; calls are re-entrant.  The one exception is moe_route_noalloc, which takes no
 *     workspace and uses a fixed device array of the library instead (see there).
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue work
 *     on it and return; nothing synchronises the host and no count leaves the device.
 *   - Validation: arguments are checked on the host only.  Device contents are preconditions:
 *     inputs finite, expert ids in [-1, E), a token's valid ids distinct.  Ids outside
 *     [0, E) are treated as "not routed here".
 *   - Errors: a negative MOE_ERR_* code is returned and nothing is enqueued; MOE_ERR_HIP means
 *     a launch failed (moe_status_string() then names the HIP error).
 *   - Shapes (MOE_ERR_SHAPE otherwise): T >= 0, 1 <= E <= 1024, 1 <= k <= min(E, 64),
 *     d and f positive multiples of 128 (MOE_FP8_E4M3, MOE_MXFP8: of 256) and at most 65536,
 *     T*k < 2^31 (MOE_MXFP8: T*k + 127*E rounded up to 128 < 2^31).
 *   - fp8 (MOE_FP8_E4M3): codes are OCP e4m3 (bias 7, max 448, no infinities); a block's value
 *     is code * scale with its fp32 scale ([Prime] "Mit csinált a Prime Intellect?": blockwise
 *     FP8 is one of the kernel's data types).  Outputs and gradients stay bf16/fp32.
 *   - MXFP8 (MOE_MXFP8): x, W1, W2 are passed in bf16 (the 16-bit master copies) and the
 *     library quantises them on every call to OCP MXFP8 (e4m3 codes, one E8M0 exponent per 32
 *     values along each GEMM's K; [JAX] "Csoportosított mátrixszorzás és összevont
 *     adatmozgatás": group-aware MXFP8 quantisation feeding an MXFP8 grouped GEMM; [TE]
 *     "צמצום הזיכרון ותקורות הכימות": one scale per 32 values).  The exponent of a block is the
 *     smallest power of two that brings its maximum magnitude within 448 (no clipping); elements
 *     round to nearest even.  The data-gradient GEMMs use weights quantised along their own K;
 *     moe_forward produces both quantisations in one pass over each weight matrix and keeps
 *     the backward's in `saved`.  Weight gradients run in MXFP8 too, quantised along their K,
 *     the token axis (see moe_backward).  d and f must be multiples of 256.
 *   - Alignment (MOE_ERR_ALIGN otherwise): tensors 16-byte aligned, ws and saved 256-byte
 *     aligned (every torch/hipMalloc allocation is).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_BF16 = 0, MOE_FP8_E4M3 = 1, MOE_MXFP8 = 2 } moe_dtype;

typedef struct {
  int64_t T, d, f, E, k;
  int32_t dtype; /* moe_dtype */
  int32_t reserved; /* must be 0 */
} moe_dims;

enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,      /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,     /* dims outside the supported range */
  MOE_ERR_DTYPE = -3,     /* dtype not supported by this call */
  MOE_ERR_WORKSPACE = -4, /* ws_bytes smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = -5,       /* a HIP launch failed */
  MOE_ERR_ALIGN = -6      /* a device buffer is not 16-byte aligned (ws and saved: 256) */
};

enum { MOE_WS_ROUTE = 0, MOE_WS_FORWARD = 1, MOE_WS_BACKWARD = 2, MOE_WS_ROUTER = 3 };

/* Workspace bytes needed by moe_route/moe_plan (which = MOE_WS_ROUTE), moe_forward
 * (MOE_WS_FORWARD), moe_backward (MOE_WS_BACKWARD) or moe_router_backward (MOE_WS_ROUTER).
 * Host only. */
int moe_workspace_bytes(const moe_dims* dims, int which, size_t* out);

/* Bytes of the `saved` context moe_forward writes and moe_backward reads (the GEMM1 output
 * H = [gate | up] and the scaled SwiGLU activations).  Host only. */
int moe_saved_bytes(const moe_dims* dims, size_t* out);

/* Top-k routing plus the expert plan.  Per token: the k largest logits (descending, ties to
 * the lower expert id) and topk_w = softmax over those k logits in fp32 ([JAX] "A dropless MoE
 * minden tokent feldolgoz": a learned router activates only the top-K experts per token).
 * Then counts, offsets, perm and inv_perm as for moe_plan. */
int moe_route(const moe_dims* dims, const float* logits, int32_t* topk_ids, float* topk_w,
              int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
              void* ws, size_t ws_bytes, void* stream);

/* moe_route without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same outputs,
 * bit for bit.  The plan's tables live in a fixed 4 MiB device array inside the library, one per
 * GPU, held until the process ends; every shape this header accepts fits it (MOE_ERR_WORKSPACE
 * otherwise).  The call allocates nothing.  All calls on one GPU share that array, so calls that
 * overlap in time on one GPU (different streams, or different host threads) race and must be
 * serialised by the caller; calls on one stream are ordered and safe.  The first call on a GPU
 * looks up the array's device address (MOE_ERR_HIP if that fails). */
int moe_route_noalloc(const moe_dims* dims, const float* logits, int32_t* topk_ids, float* topk_w,
                      int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* stream);

/* Expert plan for already-routed pairs: per-expert counts, their exclusive prefix sum and the
 * stable counting sort of pairs by expert (ragged per-expert groups: [JAX] "Az egyenetlen
 * terhelés lassítja a tanítást" [uneven load slows training]; per-expert counts as split
 * sizes: [TE] "מומחים מקובצים במקום לולאת Python" [grouped experts instead of a Python loop]).
 * Integer only, bit-exact and deterministic.  Ids -1 are skipped (inv_perm = -1). */
int moe_plan(const moe_dims* dims, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
             int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);

/* Forward: y[t] = sum_j w[t,j] * (silu(x_t W1[e] gate) * (x_t W1[e] up)) W2[e], e = ids[t,j],
 * over routed slots ([Mega] "Mega MoE คืออะไร?" [what is Mega MoE?]: dispatch, two linear layers,
 * SwiGLU, combine; [TE] "צמצום הזיכרון ותקורות הכימות": GroupedLinear -> ScaledSwiGLU ->
 * GroupedLinear).  The token gather is fused into the first grouped GEMM's operand loads, the
 * routing weight into its SwiGLU epilogue, and the combine sums a token's k per-pair outputs in
 * fp32 in slot order with one bf16 rounding.  Each expert is computed at its real row count
 * ([JAX] "Csoportosított mátrixszorzás és összevont adatmozgatás" [grouped GEMM and fused data
 * movement]).  `saved` (moe_saved_bytes) receives what moe_backward needs.  For
 * dtype = MOE_FP8_E4M3 the *_scale arguments are required when T > 0 (MOE_ERR_NULL); for bf16
 * they must be NULL (MOE_ERR_DTYPE).  fp8: both grouped GEMMs run on e4m3 operands with fp32
 * accumulation and per-128-K scale promotion; the scaled SwiGLU output feeding the second one
 * is requantised to e4m3 with one scale (its absolute maximum / 448) per row per 128 columns
 * ([TE] "צמצום הזיכרון ותקורות הכימות" [reducing memory and quantisation overheads]). */
int moe_forward(const moe_dims* dims, const void* x, const float* x_scale,
                const void* W1, const float* W1_scale, const void* W2, const float* W2_scale,
                const float* topk_w, const int32_t* offsets, const int32_t* perm,
                const int32_t* inv_perm, void* y, void* saved, void* ws, size_t ws_bytes,
                void* stream);

/* The bf16 moe_forward with the dispatch gather, both grouped GEMMs and the scaled SwiGLU in one
 * persistent launch fed by a device work queue, followed by the combine ([Mega] "Mega MoE
 * คืออะไร?" [what is Mega MoE?]: dispatch, the two linear layers and SwiGLU fused into one
 * kernel).  Same arguments, results and `saved` contents as moe_forward with dtype MOE_BF16 and
 * NULL scales, so moe_backward accepts its `saved`; y, H and As are bitwise equal to
 * moe_forward's.  A work item is a row tile (256 sorted rows of one expert): its block runs the
 * up product over all of f, then the down product over all of d for the same rows, so the work
 * is coarser than moe_forward's per-tile launches (slower when the row tiles are few against the
 * compute units).  Blocks take items with atomic adds on counters in `ws` and never wait for
 * one another; `ws` needs moe_workspace_bytes(MOE_WS_FORWARD).  dtype other than MOE_BF16:
 * MOE_ERR_DTYPE.  Other errors as moe_forward. */
int moe_forward_fused(const moe_dims* dims, const void* x, const void* W1, const void* W2,
                      const float* topk_w, const int32_t* offsets, const int32_t* perm,
                      const int32_t* inv_perm, void* y, void* saved, void* ws, size_t ws_bytes,
                      void* stream);

/* Backward of moe_forward for L = sum(dy * y) ([Prime] "Mit csinált a Prime Intellect?" [what
 * did Prime Intellect do?]: a backward pass for the fused MoE kernel).  Writes dx (bf16),
 * dW1 and dW2 (bf16; an expert with no routed pair gets exactly zero), d_topk_w (fp32, 0 on
 * unrouted slots) and, if d_logits is not NULL, d_logits[t, ids[t,j]] =
 * w[t,j] * (d_topk_w[t,j] - sum_i w[t,i] d_topk_w[t,i]) and 0 elsewhere (the softmax over the
 * kept logits; topk_ids is then required).  `saved` must come from moe_forward on the same
 * inputs.  Every reduction has a fixed order, so results are bitwise reproducible.
 * fp8 (MOE_FP8_E4M3): dy is quantised like the forward activations (1x128 blocks) for the two
 * data-gradient GEMMs and dH is requantised the same way between them.  The weight gradients
 * dW2 = As^T dy and dW1 = x^T dH run as bf16 GEMMs with fp32 accumulation on the bf16 dy, the
 * layer's own bf16 As and dH, and x dequantised once to bf16 (code * scale in fp32, one
 * rounding): their K is the token axis, which the 1x128 blocks of the inputs do not follow.
 * MXFP8 (MOE_MXFP8): the weight gradients run as MXFP8 GEMMs whose K is the expert's rows; both
 * operands are quantised in blocks of 32 consecutive sorted rows that never straddle two experts
 * ([JAX] "Csoportosított mátrixszorzás és összevont adatmozgatás": group-aware quantisation). */
int moe_backward(const moe_dims* dims, const void* dy, const void* x, const float* x_scale,
                 const void* W1, const float* W1_scale, const void* W2, const float* W2_scale,
                 const int32_t* topk_ids, const float* topk_w, const int32_t* offsets,
                 const int32_t* perm, const int32_t* inv_perm, const void* saved, void* dx,
                 void* dW1, void* dW2, float* d_topk_w, float* d_logits, void* ws,
                 size_t ws_bytes, void* stream);

/* Router scores (the gate in front of moe_route): logits[T, E] = x[T, d] . Wg[d, E] with bf16 x and
 * gate weight Wg (row-major [d, E]), fp32 accumulation and fp32 output ([JAX] "A dropless MoE
 * minden tokent feldolgoz": a learned router scores the experts and keeps the top K).  Feeding
 * these logits to moe_route gives the layer's routing.  dtype MOE_BF16 or MOE_MXFP8 (x is bf16 in
 * both; MOE_FP8_E4M3: MOE_ERR_DTYPE).  x, Wg and logits 16-byte aligned; T = 0 does nothing. */
int moe_router_logits(const moe_dims* dims, const void* x, const void* Wg, float* logits, void* stream);

/* Backward through moe_router_logits for the layer's d_logits [T, E] (fp32, as moe_backward writes
 * it).  dWg = x^T . d_logits (bf16 [d, E], fp32 accumulation) when dWg is not NULL: the token axis
 * is cut into slices whose fp32 partial sums live in `ws` (moe_workspace_bytes(MOE_WS_ROUTER)) and
 * are added in slice order, so the result is bitwise reproducible; an empty layer (T = 0) writes
 * zeros.  When dx is not NULL, the part of the input gradient that flows through the logits is
 * added to it in place: dx[t] = bf16(dx[t] + sum_e d_logits[t, e] Wg[:, e]), the sum in fp32 and
 * one rounding (pass moe_backward's dx to get the whole input gradient of the routed layer).
 * d_logits enters the MFMA rounded to bf16.  Same dtype, alignment and workspace rules as the
 * other calls (ws 256-byte aligned). */
int moe_router_backward(const moe_dims* dims, const void* x, const void* Wg, const float* d_logits,
                        void* dx, void* dWg, void* ws, size_t ws_bytes, void* stream);

/* Dispatch on its own (bf16): for every slot with pos = inv_perm[t*k+j] >= 0, xp[pos] = x[t]
 * (so xp[pos] = x[perm[pos] / k] for pos < offsets[E]); rows of xp at or past offsets[E] are left
 * untouched.  Token-major: each row of x is read once and written to its k positions.  xp is
 * bf16 [T*k, d].  ([JAX] "Csoportosított mátrixszorzás és összevont adatmozgatás": dispatch
 * sends tokens to their experts.)  The forward pass does not call it (its GEMM gathers rows
 * directly); it exists for callers that want expert-sorted activations. */
int moe_permute(const moe_dims* dims, const void* x, const int32_t* inv_perm, void* xp, void* stream);

/* Combine on its own (bf16): y[t] = sum over j = 0..k-1 with inv_perm[t*k+j] >= 0 of
 * op[t*k+j], summed in fp32 in ascending j and rounded once to bf16 (combine gathers the
 * results back and restores token order: [JAX] "Az egyenetlen terhelés lassítja a
 * tanítást").  op is bf16 [T*k, d] in pair (slot) order. */
int moe_combine(const moe_dims* dims, const void* op, const int32_t* inv_perm, void* y,
                void* stream);

/* Optional profiling hook (process-wide; none by default).  When set, each call invokes
 * hook(stage, 1, stream, user) on the calling thread right before it enqueues a stage's kernel
 * and hook(stage, 0, stream, user) right after, so a profiler can record stream events around
 * every kernel.  `stage` is a static string naming the kernel ("gemm_up", "combine", ...).
 * Pass NULL to remove the hook.  Setting it while another thread is inside a call races. */
typedef void (*moe_stage_hook)(const char* stage, int begin, void* stream, void* user);
int moe_set_stage_hook(moe_stage_hook hook, void* user);

/* MXFP8 quantisation on its own (the same kernels the MOE_MXFP8 path runs).  src is bf16
 * [batch, rows, cols] (row-major).  block_axis = 1: each block is 32 consecutive values of a row
 * (cols % 32 == 0), exps is [batch, rows, cols/32]; block_axis = 0: each block is 32
 * consecutive rows of one column (rows % 32 == 0, cols % 8 == 0), exps is [batch, rows/32,
 * cols].  codes (e4m3) has src's shape; exps are E8M0 bytes (2^(E-127)).  Rules as for
 * MOE_MXFP8 above.  Tensors 16-byte aligned.  ([JAX] "Csoportosított mátrixszorzás és
 * összevont adatmozgatás": group-aware MXFP8 quantisation.) */
int moe_mxfp8_quantize(const void* src, int64_t batch, int64_t rows, int64_t cols, int block_axis, void* codes,
                       void* exps, void* stream);

/* The MOE_MXFP8 path's weight quantiser on its own: one read of bf16 src [batch, rows, cols]
 * (row-major; rows % 32 == 0, cols % 256 == 0) writes both orientations of each matrix.
 * col_codes / col_exps: blocks of 32 consecutive rows of one column, exponents [batch, rows/32,
 * cols] (as block_axis = 0 above).  row_codes / row_words: blocks of 32 consecutive values of a
 * row, with the exponents as 32-bit words by 128-column step, [batch, cols/128, rows] words:
 * word (t, r) holds the E8M0 bytes of blocks 4t .. 4t+3 of row r (byte j for block 4t + j), the
 * layout the MXFP8 GEMMs read.  Codes have src's shape.  src and the codes 16-byte aligned,
 * col_exps 8-byte aligned, row_words 4-byte aligned.  ([JAX] "Csoportosított mátrixszorzás és
 * összevont adatmozgatás": MXFP8 blocks along each product's K; a weight matrix is the K operand
 * of the forward along its rows and of the data gradient along its columns.) */
int moe_mxfp8_quantize_weights(const void* src, int64_t batch, int64_t rows, int64_t cols, void* col_codes,
                               void* col_exps, void* row_codes, void* row_words, void* stream);

/* Static string for a status code (for MOE_ERR_HIP: the last HIP error on this thread). */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
