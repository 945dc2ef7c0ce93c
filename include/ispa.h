/*
 * ispa.h — C ABI of the ISPA hot path on AMD MI355X (gfx950).
 *
 * Instance-Specific Parametric Absorption converts some full-attention layers
 * of an autoregressive video model to local attention after a short warmup,
 * absorbing the lost history into the attention output projection.  This
 * library implements the warmup's dual-stream attention and the closed-form
 * absorb that follows it:
 *
 *   ispa_decomp_attn   local and historical attention branches plus their
 *                      log-sum-exp merge (A_loc and A_full rows),
 *   ispa_decomp_attn_noalloc   the same with its scratch in a static device
 *                      array (no workspace argument, nothing allocated),
 *   ispa_decomp_attn_segments  the same over a list of K/V segments
 *                      (sink, chunk, history pages) attended in place,
 *   ispa_decomp_attn_splitkv   the same with the keys split across
 *                      workgroups (even load) and merged through LSE,
 *   ispa_gram_accum    G = A_loc^T A_loc, C = A_loc^T (A_full - A_loc) and
 *                      E = (A_full - A_loc)^T (A_full - A_loc),
 *   ispa_absorb_solve  dW = (G + lambda I)^-1 C W  (Cholesky + triangular solves),
 *   ispa_layer_eps     the post-fit reconstruction error used to rank layers,
 *   ispa_select_layers the k lowest-error layers (those converted),
 *   ispa_absorb_apply  W += dW for the converted layers,
 *   ispa_decomp_attn_fp8k, ispa_quantize_fp8_*, ispa_w8a8_gemm
 *                      fp8 keys / queries and the W8A8 projection,
 *   ispa_fit_error, ispa_lambda_from_trace, ispa_absorb_solve_lambdas, ispa_absorb_solve_ex,
 *   ispa_select_layers_below, ispa_gather_layers, ispa_absorb_apply_compact
 *                      selection and lambda variants (error before the fit or
 *                      on held-out rows, lambda from tr(G), threshold K),
 *   ispa_full_attn     one softmax pass over all keys (the comparison pass),
 *   ispa_lse_merge     standalone N-way merge of (O, LSE) partial results.
 *
 * Sources: "Technical Summary: Instance-Specific Parametric Absorption (ISPA)
 * for Memory-Efficient Video Generation" (gist.science), section 2
 * "Methodology" (Dual-Stream Warmup, Layer Absorb, Memory-Efficient Inference,
 * Dynamic Layer Selection) and section 3 "Key Contributions" (online softmax);
 * "Towards Memory-Efficient Autoregressive Video Generation via
 * Instance-Specific Parametric Absorption" (mlsanity.com), "Abstract (arXiv)".
 *
 * Conventions for every call
 * --------------------------
 * - Every buffer is DEVICE memory owned by the caller.  The library never
 *   allocates or frees in these calls; scratch space is a caller-provided
 *   workspace whose size is queried first.  Its contents on entry do not
 *   matter (a call reads only workspace bytes it has written itself); calls
 *   that share a workspace must not run concurrently.
 * - Calls only enqueue work on `stream` (a hipStream_t; NULL = default
 *   stream) and return; results are valid once the stream is synchronised.
 *   The library creates no streams or events and keeps no state between
 *   calls besides its loaded kernels.  ispa_absorb_solve_ex can also use a
 *   second stream the CALLER owns (ispa_side_stream_t), forked from and joined
 *   back to `stream` with the caller's events inside the call, so the call
 *   stays ordered on `stream` and can be captured into a graph.
 * - Inputs must not alias outputs (the one exception is W_new == W).
 * - Layouts: Q, K, V and O are [tokens, heads, head_dim] contiguous, so an O
 *   buffer is also the row-major [tokens, d] matrix A with d = heads*head_dim
 *   and column h*head_dim + e.  LSE is [heads, tokens] float32, natural log,
 *   scale included.  G, C, E, W, dW, W_new are row-major float32.
 * - bf16 tensors are passed as 16-bit patterns (uint16 storage).
 * - Return value: ISPA_OK, or an error status with detail in
 *   ispa_last_error() (thread-local).  Nothing throws, aborts or exits.
 *   Validation errors are returned before anything is enqueued.
 * - Non-finite inputs propagate (a NaN in a Q row makes that row's outputs
 *   NaN); they are not checked.
 */
#ifndef ISPA_H
#define ISPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ISPA_OK = 0,
  ISPA_E_INVALID_ARG = 1, /* null required pointer, bad size, misaligned pointer, unsupported shape */
  ISPA_E_UNSUPPORTED = 2, /* the current device is not gfx950 */
  ISPA_E_WORKSPACE = 3,   /* workspace missing or smaller than the queried size */
  ISPA_E_HIP = 4          /* a HIP runtime / launch error */
} ispa_status_t;

typedef enum { ISPA_F32 = 0, ISPA_BF16 = 1 } ispa_dtype_t;

/* Shape of one attention call.  Q and each output ([n_q, H, D]), the keys
 * and values ([n_loc + n_hist, H, D] in all) and each LSE ([H, n_q]) must hold
 * fewer than 2^31 elements; a larger shape returns ISPA_E_INVALID_ARG. */
typedef struct {
  int32_t heads;    /* H >= 1 */
  int32_t head_dim; /* D in {64, 128} */
  int64_t n_q;      /* queries, >= 0 */
  int64_t n_loc;    /* local keys (sink rows then current-chunk rows), >= 1 */
  int64_t n_hist;   /* history keys, >= 0; 0 = local-attention (L-layer) mode */
  float scale;      /* softmax scale, usually 1/sqrt(head_dim); > 0 */
  int32_t dtype;    /* ispa_dtype_t of Q, K, V and O */
} ispa_attn_desc_t;

/*
 * ispa_decomp_attn — decomposable attention of one chunk (one launch).
 *
 * Source: ISPA technical summary, section 2 "Methodology", step 1
 * "Dual-Stream Warmup": the local stream attends to the current chunk plus the
 * sink tokens, the full stream to the entire context; the decomposable form
 * runs a local and a historical branch, each an online-softmax pass that keeps
 * its log-sum-exp state, and fuses them afterwards.  Reading used: scores are
 * scale*<q,k> with no mask; the merge is LSE = logaddexp(LSE_loc, LSE_hist),
 * O_full = e^(LSE_loc-LSE) O_loc + e^(LSE_hist-LSE) O_hist, and is computed in
 * the history branch's epilogue from the float32 branch outputs (O_loc is
 * parked in the workspace between the branches), so O_full is rounded once.
 *
 *   Q       [n_q,  H, D]      K_loc, V_loc [n_loc, H, D]   K_hist, V_hist [n_hist, H, D]
 *   O_loc, O_hist, O_full [n_q, H, D] (dtype)   LSE_* [H, n_q] float32
 *
 * Every output pointer may be NULL (that output is not written).  With
 * n_hist == 0, K_hist/V_hist are ignored, LSE_hist = -inf, O_hist = 0, and
 * O_full is bitwise equal to O_loc.  Pointers must be 16-byte aligned.
 * `workspace` (device, >= ispa_decomp_attn_workspace_size bytes) is required
 * when O_full is requested with n_hist > 0 in bf16, else may be NULL;
 * ISPA_E_WORKSPACE otherwise.
 * dtype BF16 computes QK^T and PV on bf16 matrix cores with float32
 * accumulation and float32 softmax state; F32 computes everything in float32.
 */
ispa_status_t ispa_decomp_attn(const ispa_attn_desc_t* desc, const void* Q, const void* K_loc,
                               const void* V_loc, const void* K_hist, const void* V_hist, void* O_loc,
                               float* LSE_loc, void* O_hist, float* LSE_hist, void* O_full,
                               float* LSE_full, void* workspace, size_t workspace_bytes, void* stream);

/* Scratch bytes ispa_decomp_attn_noalloc keeps in device memory (per GPU). */
#define ISPA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * ispa_decomp_attn_noalloc — ispa_decomp_attn without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 *
 * The only scratch the call needs, the float32 O_loc the merge reads back
 * (n_q * heads * head_dim * 4 bytes when O_full is requested in bf16 with
 * history keys), lives in a static device array of ISPA_NOALLOC_SCRATCH_BYTES
 * (128 MiB) that each GPU the library runs on holds until the process ends;
 * the call allocates nothing.  A shape that needs more returns
 * ISPA_E_INVALID_ARG before anything is enqueued (128 MiB covers n_q = 4680
 * queries at 40 heads x 128).  The scratch needs no clearing (each value is
 * read back only by the lane that wrote it in the same launch).  Calls that
 * overlap on one GPU (two streams, or two host threads) share the array and
 * race: serialise them.  Arguments, outputs and the other errors are those of
 * ispa_decomp_attn; results are bitwise equal to it.
 */
ispa_status_t ispa_decomp_attn_noalloc(const ispa_attn_desc_t* desc, const void* Q, const void* K_loc,
                                       const void* V_loc, const void* K_hist, const void* V_hist, void* O_loc,
                                       float* LSE_loc, void* O_hist, float* LSE_hist, void* O_full,
                                       float* LSE_full, void* stream);

/* At most this many K/V segments per ispa_decomp_attn_segments call. */
#define ISPA_MAX_KV_SEGMENTS 16

/* One contiguous run of cached keys and values: K, V [n_rows, H, D] (dtype). */
typedef struct {
  const void* K;
  const void* V;
  int64_t n_rows; /* >= 1 */
} ispa_kv_segment_t;

/*
 * ispa_decomp_attn_segments — ispa_decomp_attn over keys given as a list of
 * segments instead of one K_loc and one K_hist buffer (one launch).
 *
 * Source: ISPA technical summary, section 2 "Methodology": step 1 (the local
 * stream sees the sink tokens plus the current chunk, the full stream the
 * whole context) and step 3 (a converted layer drops its history K/V while
 * the sink stays); the streaming generation appends every finished chunk's
 * keys to the history.  A cache kept as separate buffers (a sink buffer, the
 * current chunk, history pages or a wrapped ring buffer) is attended in place,
 * with no concatenation copy.
 *
 * segs[0 .. n_loc_segs-1] are the local branch's keys, segs[n_loc_segs ..
 * n_segs-1] the history branch's, in order; `segs` is a HOST array read
 * during the call.  1 <= n_loc_segs <= n_segs <= ISPA_MAX_KV_SEGMENTS; every
 * segment has n_rows >= 1 and 16-byte aligned K, V; the local rows must add
 * up to desc->n_loc and the history rows to desc->n_hist (ISPA_E_INVALID_ARG
 * otherwise).  Within a branch the softmax is over the union of its segments,
 * so results depend on the keys, not on how they are split; the order of
 * floating-point accumulation follows the segments, so a different split of
 * the same keys may round differently.  Outputs, workspace and errors are
 * those of ispa_decomp_attn (same workspace size for the same desc).
 */
ispa_status_t ispa_decomp_attn_segments(const ispa_attn_desc_t* desc, const void* Q,
                                        const ispa_kv_segment_t* segs, int32_t n_segs, int32_t n_loc_segs,
                                        void* O_loc, float* LSE_loc, void* O_hist, float* LSE_hist,
                                        void* O_full, float* LSE_full, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* At most this many workgroups per ispa_decomp_attn_splitkv call. */
#define ISPA_MAX_SPLITKV_WORKERS 65535

/*
 * ispa_decomp_attn_splitkv — ispa_decomp_attn_segments with the keys of every
 * (head, query tile) split into P equal pieces on P workgroups (split-KV),
 * for shapes whose (head, query tile) units would leave most of the GPU idle
 * (few heads, short query chunks, long histories); two launches: attention,
 * then a merge of the pieces.
 *
 * Source: ISPA technical summary, section 2 "Methodology", step 1 (branches
 * are independent online-softmax passes whose log-sum-exp states combine
 * exactly afterwards) and section 3 (online softmax).  The same identity
 * that fuses the local and history branches fuses any partition of a branch's
 * keys: a piece of a branch leaves (O_p, LSE_p), and O = sum_p
 * e^(LSE_p - LSE) O_p with LSE = log sum_p e^(LSE_p).
 *
 * `n_workers` workgroups (0 = one per compute unit of the current device,
 * <= ISPA_MAX_SPLITKV_WORKERS).  The units (256 queries of one head) are dealt
 * to the 8 XCDs in contiguous blocks; P is the number of workgroups every XCD
 * can give each of its units (at most the number of 128-key tiles).  With
 * P = 1 the call is ispa_decomp_attn_segments exactly (bitwise).  Otherwise
 * every piece leaves float32 partial states in the workspace and the second
 * launch merges them (float32, outputs rounded once); results equal the
 * unsplit call's up to rounding (tested against the float64 reference).
 * BF16 only (ISPA_E_INVALID_ARG for F32).  Arguments, outputs and errors are
 * those of ispa_decomp_attn_segments; `workspace` (device, >=
 * ispa_decomp_attn_splitkv_workspace_size(desc, n_workers) bytes) is always
 * required (ISPA_E_WORKSPACE otherwise).
 */
ispa_status_t ispa_decomp_attn_splitkv(const ispa_attn_desc_t* desc, const void* Q,
                                       const ispa_kv_segment_t* segs, int32_t n_segs, int32_t n_loc_segs,
                                       int32_t n_workers, void* O_loc, float* LSE_loc, void* O_hist,
                                       float* LSE_hist, void* O_full, float* LSE_full, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Workspace bytes of ispa_decomp_attn_splitkv: the merge's float32 O_loc
 * (with history keys, rounded up to 256 bytes) plus one partial slot of
 * 2*BM*(D+1) float32 per workgroup (BM = 256 queries; 264 KB at D = 128).
 * n_workers = 0 sizes for the current device (0 if there is none).
 * Support call: no passage of the pages defines it. */
size_t ispa_decomp_attn_splitkv_workspace_size(const ispa_attn_desc_t* desc, int32_t n_workers);

/* Workspace bytes ispa_decomp_attn needs for this shape: n_q*H*D*4 for bf16
 * with history keys (the float32 O_loc the merge reads), else 0.  Needed only
 * when O_full is requested.
 * Support call: no passage of the pages defines it. */
size_t ispa_decomp_attn_workspace_size(const ispa_attn_desc_t* desc);

/*
 * ispa_full_attn — one online-softmax pass over n_loc + n_hist keys given as a
 * single concatenated K, V ([n_loc + n_hist, H, D]).  This is the
 * single-stream attention the decomposable pass is compared against (same
 * kernel family, one phase).  O / LSE may be NULL.
 * Source: ISPA technical summary, section 2 "Methodology", step 1 (the full
 * stream, here over the keys concatenated) and section 3 (online softmax).
 */
ispa_status_t ispa_full_attn(const ispa_attn_desc_t* desc, const void* Q, const void* K, const void* V,
                             void* O, float* LSE, void* stream);

/*
 * ispa_lse_merge — merge n_parts partial attention results over disjoint key
 * sets into the result over their union: LSE = log sum_p exp(LSE_p),
 * O = sum_p exp(LSE_p - LSE) O_p.  Source: ISPA technical summary, section 2,
 * step 1 (branches fused after the fact from their LSE states).
 * O_parts / LSE_parts are HOST arrays of n_parts DEVICE pointers
 * (O_p [n_q,H,D] dtype, LSE_p [H,n_q] float32).  1 <= n_parts <= 16.
 * A part with LSE = -inf contributes nothing.  LSE_out may be NULL.
 */
ispa_status_t ispa_lse_merge(int32_t n_parts, const void* const* O_parts, const float* const* LSE_parts,
                             int64_t n_q, int32_t heads, int32_t head_dim, int32_t dtype, void* O_out,
                             float* LSE_out, void* stream);

/* Workspace bytes ispa_gram_accum needs for these sizes (0 for float32 or no
 * rows): the bf16 split of D for one block of up to 32768 rows, a counter per
 * output tile, and the split partials when rows are split over workgroups.
 * Support call: no passage of the pages defines it. */
size_t ispa_gram_workspace_size(int64_t n_rows, int32_t d, int32_t dtype);

/*
 * ispa_gram_accum — stream warmup rows into the absorb's sufficient statistics.
 *
 * Source: ISPA technical summary, section 2, step 2 "Layer Absorb": the
 * closed form needs only A_loc^T A_loc and A_loc^T (A_full - A_loc) over the
 * warmup rows; "Dynamic Layer Selection" ranks layers by the fit's error,
 * which also needs (A_full - A_loc)^T (A_full - A_loc).  With D = A_full -
 * A_loc (exact in float32 for bf16 rows):
 *   G (+)= A_loc^T A_loc,  C (+)= A_loc^T D,  E (+)= D^T D  (E optional).
 * C and E are formed from D itself, not as differences of products, so they
 * keep their accuracy when the two streams nearly agree (bf16: D enters the
 * matrix cores as two bf16 terms, D_hi + D_lo, within 2^-17 of D).
 *
 *   A_loc, A_full [n_rows, d] (dtype), row-major (an O buffer of
 *   ispa_decomp_attn is such a matrix).  G, C, E [d, d] float32.
 *   accumulate = 0 overwrites G, C (and E); 1 adds to them.
 *   E may be NULL (not formed).  G and E are written in full (both triangles
 *   hold the same bits).  d must be a multiple of 128 (bf16) or 64 (float32);
 *   0 <= n_rows with n_rows * d < 2^40 (0 rows with accumulate = 0 writes
 *   zeros).  bf16 needs `workspace` (>= ispa_gram_workspace_size bytes;
 *   ISPA_E_WORKSPACE otherwise).  The result is deterministic: no
 *   floating-point atomics, fixed reduction order.
 */
ispa_status_t ispa_gram_accum(int64_t n_rows, int32_t d, int32_t dtype, const void* A_loc,
                              const void* A_full, float* G, float* C, float* E, int32_t accumulate,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes ispa_absorb_solve needs for these sizes.
 * Support call: no passage of the pages defines it. */
size_t ispa_absorb_workspace_size(int32_t d, int32_t d_out, int32_t batch);

/*
 * ispa_absorb_solve — closed-form absorb for `batch` layers.
 *
 * Source: ISPA technical summary, section 2, step 2 "Layer Absorb" (ridge
 * objective and its closed-form minimiser, non-iterative) and step 3
 * "Memory-Efficient Inference" (W_new = W + dW).  Computes, per batch entry,
 * M = G + lambda I, M = L L^T (blocked Cholesky, float32), R = C W,
 * L Y = R, L^T dW = Y (through the explicit L^-1), then one refinement
 * step: r = R - (G + lambda I) dW formed far beyond float32 accuracy (exact
 * int8 digit-slice products for d, d_out multiples of 128, else float64
 * accumulation), dW += M^-1 r.
 *
 *   G, C [batch, d, d]; W [batch, d, d_out]; dW [batch, d, d_out]; all float32.
 *   W_new [batch, d, d_out] may be NULL or equal to W (in-place absorb).
 *   info [batch] int32 DEVICE: 0 = success; k > 0 = the leading minor of
 *   order k of G + lambda I is not positive definite (LAPACK potrf
 *   convention); then dW[b] is all NaN and W_new[b] is left untouched.
 *   G and C are read only (the factor lives in the workspace).
 *   d and d_out must be multiples of 64; lambda >= 0; batch >= 1.
 */
ispa_status_t ispa_absorb_solve(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                                const float* W, float lambda, float* dW, float* W_new, int32_t* info,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes ispa_layer_eps needs.
 * Support call: no passage of the pages defines it. */
size_t ispa_eps_workspace_size(int32_t d, int32_t d_out, int32_t batch);

/*
 * ispa_layer_eps — reconstruction error of each absorbed layer, for ranking.
 *
 * Source: ISPA technical summary, section 2 "Dynamic Layer Selection" (layers
 * ranked by reconstruction error after warmup, lowest converted).  Reading:
 * eps = ||A_loc (W + dW) - A_full W||_F^2 over the warmup rows (the lambda
 * term excluded), evaluated from the statistics of ispa_gram_accum (D =
 * A_full - A_loc; G, C, E) and the normal equation (G + lambda I) dW = C W:
 *   eps = <E W, W> - <dW, C W> - lambda ||dW||^2,
 *   eps_rel = eps / <(G + C + C^T + E) W, W>  (= eps / ||A_full W||_F^2).
 * Products in float32, the inner products reduced in float64.
 *   G, C, E [batch, d, d]; W, dW [batch, d, d_out]; eps_abs, eps_rel
 *   [batch] float64 DEVICE.
 */
ispa_status_t ispa_layer_eps(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                             const float* E, const float* W, const float* dW, float lambda,
                             double* eps_abs, double* eps_rel, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * ispa_select_layers — choose the k layers to convert to local attention.
 *
 * Source: ISPA technical summary, section 2 "Dynamic Layer Selection" (all
 * layers ranked by reconstruction error after warmup; the lowest-error ones
 * are converted).  Reading: rank by eps ascending (pass eps_rel of
 * ispa_layer_eps), NaN (a failed solve) ranks last, equal values go to the
 * lower layer index; this is a strict total order, so the result is unique.
 *   eps [n_layers] float64 DEVICE; 1 <= n_layers <= 4096; 0 <= k <= n_layers.
 *   selected [k] int32 DEVICE: the chosen layer ids, lowest eps first
 *   (may be NULL when k = 0).
 *   rank [n_layers] int32 DEVICE, may be NULL: each layer's rank (0 = lowest).
 */
ispa_status_t ispa_select_layers(int32_t n_layers, const double* eps, int32_t k, int32_t* selected,
                                 int32_t* rank, void* stream);

/*
 * ispa_absorb_apply — W_l += dW_l for the selected layers.
 *
 * Source: ISPA technical summary, section 2, step 3 "Memory-Efficient
 * Inference" (the converted layers use W_new = W + dW from then on).
 *   W, dW [n_layers, d, d_out] float32 DEVICE, stacked as in
 *   ispa_absorb_solve; selected [k] int32 DEVICE layer ids (as written by
 *   ispa_select_layers), which must be distinct; an id outside
 *   [0, n_layers) is skipped.  Unselected layers are untouched.  Each sum is
 *   one float32 addition, the same value ispa_absorb_solve writes to W_new.
 */
ispa_status_t ispa_absorb_apply(int32_t d, int32_t d_out, int32_t n_layers, const int32_t* selected,
                                int32_t k, const float* dW, float* W, void* stream);

/* ---------------------------------------------------------------------------
 * fp8 (E4M3) variants.  Source: ISPA technical summary, section 4 "Results"
 * (ISPA combined with W8A8 post-training quantisation).  The pages fix no
 * format or scaling.  Reading: E4M3 with the OCP "FN" encoding (bias 7, max
 * 448, no infinities); one absmax scale per block, scale = amax / 448 in
 * float32 (1 when amax = 0); code = x / scale (float32 division) clamped to
 * +-448 and rounded to nearest, ties to even.  Codes are uint8.
 * ------------------------------------------------------------------------- */

/* Workspace bytes of ispa_quantize_fp8_heads: ceil(n_rows / 16) * heads floats.
 * Support call: no passage of the pages defines it. */
size_t ispa_quantize_fp8_heads_workspace_size(int64_t n_rows, int32_t heads);

/*
 * ispa_quantize_fp8_heads — X [n_rows, heads, head_dim] (dtype BF16 or F32)
 * to codes X8 (same layout, uint8) with one scale per head over all its rows
 * and dims: scale [heads] float32 DEVICE.  For Q and K of
 * ispa_decomp_attn_fp8k.  head_dim 64 or 128, heads * head_dim <= 16384;
 * workspace required.
 * Source: ISPA technical summary, section 4 "Results" (ISPA combined with W8A8
 * quantisation); the format and scaling are this library's reading (E4M3,
 * absmax scales).
 */
ispa_status_t ispa_quantize_fp8_heads(int64_t n_rows, int32_t heads, int32_t head_dim, int32_t dtype, const void* X,
                                      uint8_t* X8, float* scale, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * ispa_quantize_fp8_rows — X [n_rows, d] (BF16 or F32) to codes X8 [n_rows, d]
 * with one scale per row (token): scale [n_rows] float32 DEVICE.  The
 * activation side of ispa_w8a8_gemm.  d a positive multiple of 4.
 * Source: ISPA technical summary, section 4 "Results" (ISPA combined with W8A8
 * quantisation); the format and scaling are this library's reading (E4M3,
 * absmax scales).
 */
ispa_status_t ispa_quantize_fp8_rows(int64_t n_rows, int32_t d, int32_t dtype, const void* X, uint8_t* X8,
                                     float* scale, void* stream);

/*
 * ispa_quantize_fp8_cols — W [d, d_out] float32 to codes with one scale per
 * output column: scale [d_out] float32, codes written TRANSPOSED as
 * W8T [d_out, d] (each column's d codes contiguous, the operand layout of
 * ispa_w8a8_gemm).  d a positive multiple of 4.
 * Source: ISPA technical summary, section 4 "Results" (ISPA combined with W8A8
 * quantisation); the format and scaling are this library's reading (E4M3,
 * absmax scales).
 */
ispa_status_t ispa_quantize_fp8_cols(int32_t d, int32_t d_out, const float* W, uint8_t* W8T, float* scale,
                                     void* stream);

/*
 * ispa_w8a8_gemm — Y = (A8 W8) * a_scale[row] * w_scale[col] as bf16 [n, d_out]:
 * the W8A8 output projection of an absorbed layer (A = its attention output,
 * W = its W_new).  A8 [n, d] codes per row (ispa_quantize_fp8_rows), W8T
 * [d_out, d] codes per column (ispa_quantize_fp8_cols); products of codes
 * accumulate in float32 on gfx950 fp8 matrix cores.  d a multiple of 64,
 * d_out a multiple of 128, operands below 2^32 bytes.
 * Source: ISPA technical summary, section 4 "Results" (ISPA combined with W8A8
 * quantisation); the format and scaling are this library's reading (E4M3,
 * absmax scales).
 */
ispa_status_t ispa_w8a8_gemm(int64_t n, int32_t d, int32_t d_out, const uint8_t* A8, const float* a_scale,
                             const uint8_t* W8T, const float* w_scale, void* Y, void* stream);

/* One run of fp8 keys and their values: K8 [n_rows, H, D] codes with scale
 * k_scale [H] (DEVICE, as ispa_quantize_fp8_heads writes it), V [n_rows, H, D]
 * bf16. */
typedef struct {
  const void* K8;
  const float* k_scale;
  const void* V;
  int64_t n_rows; /* >= 1 */
} ispa_kv_segment_fp8k_t;

/*
 * ispa_decomp_attn_fp8k — ispa_decomp_attn_segments with fp8 queries and
 * keys: scores scale * (q_scale[h] q8) . (k_scale[h] k8) from codes Q8
 * [n_q, H, D] (scale q_scale [H] DEVICE) and per-segment K8; S = K Q^T runs
 * on the fp8 matrix cores (twice the bf16 rate), the softmax, P V and the
 * merge as in the bf16 path, V and the outputs bf16.  A K cache held as codes
 * takes half the K bytes.  desc->dtype must be ISPA_BF16; everything else as
 * ispa_decomp_attn_segments (same workspace).
 * Source: ISPA technical summary, section 4 "Results" (ISPA combined with W8A8
 * quantisation); the format and scaling are this library's reading (E4M3,
 * absmax scales).
 */
ispa_status_t ispa_decomp_attn_fp8k(const ispa_attn_desc_t* desc, const void* Q8, const float* q_scale,
                                    const ispa_kv_segment_fp8k_t* segs, int32_t n_segs, int32_t n_loc_segs,
                                    void* O_loc, float* LSE_loc, void* O_hist, float* LSE_hist, void* O_full,
                                    float* LSE_full, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Selection and lambda variants.  The pages leave the error measure, the ridge
 * weight and the number of converted layers open; these calls give the other
 * plain readings (ISPA technical summary, section 2, "Layer Absorb" and
 * "Dynamic Layer Selection").
 * ------------------------------------------------------------------------- */

/* Workspace bytes ispa_fit_error needs: 4 * batch * d * d_out float32. */
size_t ispa_fit_error_workspace_size(int32_t d, int32_t d_out, int32_t batch);

/*
 * ispa_fit_error — eps = ||A_loc (W + dW) - A_full W||_F^2 over the rows
 * whose statistics are G, C, E (as ispa_gram_accum writes them), for ANY
 * dW: rows the fit did not see (held-out error), or dW = NULL (dW = 0: the
 * discrepancy before the fit, ||(A_full - A_loc) W||^2 = <E W, W>, which
 * needs no solve).  From the statistics:
 *   eps = <E W, W> + <G dW, dW> - 2 <dW, C W>,
 *   eps_rel = eps / <(G + C + C^T + E) W, W>.
 * ispa_layer_eps is the special case where dW solves the ridge problem on the
 * same rows.  Products in float32, inner products reduced in float64.
 *   G, C, E [batch, d, d]; W, dW [batch, d, d_out] float32 (dW nullable);
 *   eps_abs, eps_rel [batch] float64 DEVICE.  d, d_out multiples of 64.
 * Source: ISPA technical summary, section 2 "Dynamic Layer Selection" (layers ranked
 * by reconstruction error; the variants here are this library's readings of it).
 */
ispa_status_t ispa_fit_error(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                             const float* E, const float* W, const float* dW, double* eps_abs,
                             double* eps_rel, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ispa_lambda_from_trace — lambdas[b] = lam_scale * tr(G_b) / d (G's mean
 * eigenvalue; the trace summed in float64): a ridge weight that scales with
 * the layer's activations, so dW does not change when both streams are
 * scaled.  G [batch, d, d] float32, lambdas [batch] float32 DEVICE;
 * lam_scale finite, >= 0.
 * Source: ISPA technical summary, section 2, step 2 "Layer Absorb" (ridge objective
 * and its closed-form solution).
 */
ispa_status_t ispa_lambda_from_trace(int32_t d, int32_t batch, const float* G, float lam_scale, float* lambdas,
                                     void* stream);

/*
 * ispa_absorb_solve_lambdas — ispa_absorb_solve with lambda read per layer
 * from the DEVICE array lambdas [batch] float32 (as ispa_lambda_from_trace
 * writes it).  Same arguments, workspace and errors otherwise; a lambda that
 * leaves G + lambda I indefinite shows up in info, not as an error.
 * Source: ISPA technical summary, section 2, step 2 "Layer Absorb" (ridge objective
 * and its closed-form solution).
 */
ispa_status_t ispa_absorb_solve_lambdas(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                                        const float* W, const float* lambdas, float* dW, float* W_new,
                                        int32_t* info, void* workspace, size_t workspace_bytes, void* stream);

/* Flag of ispa_absorb_solve_ex: skip the refinement step. */
#define ISPA_ABSORB_NO_REFINE 1

/* A second stream the caller owns, with two events the caller owns, for
 * ispa_absorb_solve_ex: R = C W runs on `stream` beside the factorisation on
 * the call's main stream, and after it the leading part of the explicit
 * inverse of the factor, beside the factorisation's last steps.  `stream`
 * (hipStream_t) must differ from the main stream and should have the default
 * priority; `ev_fork`, `ev_join` (hipEvent_t, timing may be disabled) are
 * recorded and waited on inside the call: the side stream waits for the main
 * stream's earlier work before R = C W and for the factored blocks before the
 * inverse's part, and the main stream waits for the side stream's work before
 * the solve reads it, on every return after the fork (error returns
 * included).  The result is bitwise the same as without a side stream.  Calls that share one
 * side stream and its events must be enqueued from one host thread at a time
 * (the event record / wait pairs must not interleave). */
typedef struct {
  void* stream;
  void* ev_fork;
  void* ev_join;
} ispa_side_stream_t;

/*
 * ispa_absorb_solve_ex — ispa_absorb_solve with options: lambda from the
 * DEVICE array lambdas [batch] when it is non-NULL (else the scalar lambda),
 * flags, and an optional caller-owned side stream (`side`, NULL = everything
 * on `stream`; ispa_absorb_solve and ispa_absorb_solve_lambdas run everything
 * on `stream`).  ISPA_ABSORB_NO_REFINE skips the refinement step (the accurate
 * residual and the second pair of triangular products, ~25 % of the solve at
 * d = 5120): dW is then the float32 solve, whose error grows like
 * cond(G + lambda I) * 2^-24 instead of reaching the float32 statistics'
 * own accuracy.  Same workspace and errors as ispa_absorb_solve; a `side`
 * with a NULL member, or a side stream equal to `stream`, is
 * ISPA_E_INVALID_ARG.
 * Source: ISPA technical summary, section 2, step 2 "Layer Absorb" (ridge objective
 * and its closed-form solution).
 */
ispa_status_t ispa_absorb_solve_ex(int32_t d, int32_t d_out, int32_t batch, const float* G, const float* C,
                                   const float* W, float lambda, const float* lambdas, int32_t flags, float* dW,
                                   float* W_new, int32_t* info, void* workspace, size_t workspace_bytes,
                                   const ispa_side_stream_t* side, void* stream);

/*
 * ispa_select_layers_below — convert every layer whose error is at most tau,
 * lowest first, at most k_max of them (the number converted then follows from
 * the errors instead of being fixed).  Same total order as
 * ispa_select_layers (eps ascending, ties to the lower id, NaN never chosen).
 *   eps [n_layers] float64 DEVICE; 1 <= n_layers <= 4096; 0 <= k_max <= n_layers;
 *   tau not NaN.  selected [k_max] int32 DEVICE (the first *count entries are
 *   written); count [1] int32 DEVICE; rank [n_layers] int32 DEVICE or NULL.
 * Source: ISPA technical summary, section 2 "Dynamic Layer Selection" (layers ranked
 * by reconstruction error; the variants here are this library's readings of it).
 */
ispa_status_t ispa_select_layers_below(int32_t n_layers, const double* eps, double tau, int32_t k_max,
                                       int32_t* selected, int32_t* count, int32_t* rank, void* stream);

/*
 * ispa_gather_layers — dst[s] = src[selected[s]] for s < k, each layer
 * per_layer float32 values (to solve only the chosen layers, e.g. after
 * ranking by ispa_fit_error with dW = NULL).  src [n_layers, per_layer],
 * dst [k, per_layer] DEVICE; an id outside [0, n_layers) gives a NaN layer.
 * Source: ISPA technical summary, section 2 "Dynamic Layer Selection" and step 2
 * "Layer Absorb" (only the selected layers are solved and absorbed).
 */
ispa_status_t ispa_gather_layers(int32_t n_layers, int64_t per_layer, const float* src, const int32_t* selected,
                                 int32_t k, float* dst, void* stream);

/*
 * ispa_absorb_apply_compact — W[selected[s]] += dW[s] for s < k, where dW
 * [k, d, d_out] holds only the chosen layers in selection order (the output
 * of a solve on gathered layers).  W [n_layers, d, d_out] float32 DEVICE; ids
 * distinct; an id outside [0, n_layers) is skipped.
 * Source: ISPA technical summary, section 2, step 3 "Memory-Efficient Inference"
 * (the converted layers run with W + dW).
 */
ispa_status_t ispa_absorb_apply_compact(int32_t d, int32_t d_out, int32_t n_layers, const int32_t* selected,
                                        int32_t k, const float* dW, float* W, void* stream);

/* Human-readable name of a status code (static string).
 * Support call: no passage of the pages defines it. */
const char* ispa_status_string(ispa_status_t status);

/* Detail of the last error on the calling thread ("" if none).
 * Support call: no passage of the pages defines it. */
const char* ispa_last_error(void);

/* Library version, major*10000 + minor*100 + patch.
 * Support call: no passage of the pages defines it. */
int32_t ispa_version(void);

/* ISPA_OK if `device` is a gfx950 GPU, else ISPA_E_UNSUPPORTED (or ISPA_E_HIP).
 * Support call: no passage of the pages defines it. */
ispa_status_t ispa_device_check(int32_t device);

#ifdef __cplusplus
}
#endif

#endif /* ISPA_H */
