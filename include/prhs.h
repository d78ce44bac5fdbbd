/*
 * prhs.h -- C ABI of the MI355X (gfx950) hot path of Pre-hoc Sparsity (PrHS)
 * sparse decode.
 *
 * Source: the page "Near-Oracle KV Selection via Pre-hoc Sparsity for
 * Long-Context Inference" (Gao, Wang, Tu, Zhang, Cheng, Tao; arXiv 2602.08329).
 * Per attention head and decode step the method picks a budget of N KV entries
 * (Table I: selector S, index set S_t, budget N), attends over only those
 * entries (Abstract; Table V caption: a fused sparse-attention kernel), and
 * accounts for the attention mass it keeps and drops (Table I: tau(.), delta(.)).
 * The critical-index set of one query may be shared, dilated, with temporally
 * adjacent queries (Fig. 4; Table VIII radius r; CIS block size s).
 *
 * General contract of every call
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    never frees or retains them. Inputs must stay unchanged until the work
 *    enqueued on `stream` has completed.
 *  - Every call validates its arguments on the host BEFORE any HIP call. On
 *    any error it returns a negative status, enqueues nothing and leaves every
 *    output untouched. A detail string is available from prhs_last_error()
 *    (thread-local).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *    legacy default stream), allocates no memory and does not synchronise,
 *    unless the environment variable PRHS_DEBUG_SYNC=1 is set, in which case
 *    each call synchronises its stream and reports kernel faults as
 *    PRHS_E_HIP.
 *  - The device-checked build of this library (libprhs_checked.so, compiled
 *    with PRHS_DEVICE_CHECKS) also synchronises after each call and returns
 *    PRHS_E_HIP when a kernel met a broken input contract -- an index of a
 *    given set outside [0, t), an anchor set not strictly ascending -- or a
 *    broken internal invariant; the kernels themselves behave as in the
 *    normal build (such entries are skipped) and never trap. Neither the
 *    debug synchronisation nor the checks apply to work enqueued while the
 *    stream is being captured into a graph.
 *  - Layout: q is [B, H_q, d] contiguous. K and V are [B, H_kv, t, d] with the
 *    element strides given in prhs_dims (the d axis is contiguous). Scores are
 *    fp32 [B, H_q, scores_ld]. Index sets are int32 [B, H_q, cap] plus int32
 *    counts [B, H_q]; valid entries are ascending, unique and in [0, t);
 *    entries past the count are unspecified. Per-head scalars (lse, delta,
 *    tau) are fp32 [B, H_q].
 *  - Query head h reads KV head h / G with G = H_q / H_kv (grouped-query
 *    attention).
 *  - Workspaces: a call that takes `ws` needs at least prhs_workspace_bytes()
 *    bytes, 16-byte aligned; their contents on entry do not matter. Calls
 *    that share a workspace must not run concurrently.
 *  - Alignment: q, K, V and scores base pointers must be 16-byte aligned;
 *    kv_stride_t * element size, kv_stride_h and kv_stride_b must keep every
 *    row 16-byte aligned; scores_ld must be a multiple of 4.
 */
#ifndef PRHS_H
#define PRHS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. 0 is success; every error is negative. */
enum {
  PRHS_OK = 0,
  PRHS_E_NULL = -1,      /* a required pointer is NULL                                   */
  PRHS_E_DIMS = -2,      /* H_q % H_kv != 0, t < 1, d unsupported, bad strides/ld, t too large */
  PRHS_E_DTYPE = -3,     /* unknown element type                                         */
  PRHS_E_BUDGET = -4,    /* N outside [1, t], delta target outside [0, 1], radius < 0, bad mode */
  PRHS_E_CAPACITY = -5,  /* an index buffer is smaller than the result may need           */
  PRHS_E_WORKSPACE = -6, /* workspace NULL or smaller than prhs_workspace_bytes()         */
  PRHS_E_HIP = -7,       /* the HIP runtime reported an error at launch (or at debug sync) */
  PRHS_E_ALIGN = -8      /* a pointer, stride or ld breaks the alignment rules above      */
};

/* Element type of q, K and V. Scores, outputs and mass values are always fp32. */
enum { PRHS_F32 = 0, PRHS_F16 = 1 };

/* Selection modes of prhs_select_topk. */
enum { PRHS_TOPN = 0, PRHS_DELTA = 1 };

/* Operations for prhs_workspace_bytes. */
enum { PRHS_OP_SCORE = 0, PRHS_OP_SELECT = 1, PRHS_OP_DECODE = 2, PRHS_OP_ANCHOR_STEP = 3,
       PRHS_OP_DENSE = 4, PRHS_OP_EXPAND = 5 };

/* Largest context length the selection takes (calls that select:
 * prhs_select_topk, prhs_anchor_step, prhs_adaptive_step, prhs_random_expand).
 * Up to 65536 keys a head's scores are held on chip; longer rows are searched
 * and emitted by streaming the score row, in tiles of 65536 positions. */
#define PRHS_MAX_SELECT_CTX 262144

typedef struct prhs_dims {
  int32_t batch;        /* B >= 1                                           */
  int32_t n_q_heads;    /* H_q >= 1, a multiple of n_kv_heads               */
  int32_t n_kv_heads;   /* H_kv >= 1                                        */
  int32_t head_dim;     /* d: 64 or 128                                     */
  int32_t ctx_len;      /* t >= 1: keys in the cache                        */
  int32_t dtype;        /* PRHS_F32 or PRHS_F16                             */
  int64_t kv_stride_b;  /* element strides of K and V (same layout for both) */
  int64_t kv_stride_h;
  int64_t kv_stride_t;  /* >= d                                             */
  int32_t scores_ld;    /* row stride of the scores buffer, >= t            */
} prhs_dims;

/*
 * prhs_score -- scaled dot-product scores of the decode query against every
 * cached key, and the dense log-sum-exp (Table I: q, K, d and the attention
 * weight A(.); the scale 1/sqrt(d) is the standard one).
 *
 *   scores[b,h,i] = (sum_c q[b,h,c] * K[b,h/G,i,c]) / sqrt(d)   for i < t
 *   lse_all[b,h]  = log sum_i exp(scores[b,h,i])
 *
 * Products are accumulated in fp32. The K row of every key is read once for
 * all G query heads of its group. lse_all may be NULL (then ws may be NULL).
 * ws: at least prhs_workspace_bytes(dims, PRHS_OP_SCORE, 0) bytes (per-chunk
 * partial maxima and sums).
 */
int prhs_score(const prhs_dims* dims, const void* q, const void* k, float* scores,
               float* lse_all, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * prhs_select_topk -- the per-head index set S (Table I: selector S, set S_t,
 * budget N).
 *
 * mode PRHS_TOPN: the top-k oracle (Fig. 1, Fig. 2, Fig. 9): the n_budget keys
 *   of largest score; ties at the boundary go to the lower index.
 * mode PRHS_DELTA: control of the dropped mass (Abstract): the smallest
 *   N* >= 1 whose top-N* set leaves delta = sum of the dropped weights
 *   exp(s - lse_all) <= delta_target, capped at n_budget. Needs lse_all. When
 *   the cap binds, cap_hit[b,h] = 1 (else 0) if cap_hit is not NULL.
 *   Weights are accumulated in 2^-40 fixed point, so the result does not
 *   depend on the order of accumulation.
 *
 * Output: idx[b,h,0:count) ascending; count[b,h] = N (TOPN) or N* (DELTA).
 * sel_scores (nullable, fp32 [B, H_q, idx_cap]): the scores of the selected
 * keys in the same order as idx, for prhs_sparse_decode.
 * Requires 1 <= n_budget <= t, n_budget <= idx_cap, 0 <= delta_target <= 1,
 * t <= PRHS_MAX_SELECT_CTX. Scores must be finite or -inf (NaN is outside
 * the contract); -0.0 and +0.0 compare equal. lse_all may be NULL in TOPN mode.
 */
int prhs_select_topk(const prhs_dims* dims, const float* scores, const float* lse_all,
                     int32_t mode, int32_t n_budget, float delta_target, int32_t* idx,
                     int32_t idx_cap, int32_t* count, int32_t* cap_hit, float* sel_scores,
                     hipStream_t stream);

/*
 * prhs_cis_reuse -- critical-index-set sharing with dilation (Fig. 4: the set
 * of one query serves the next queries, grown around its clusters; Table VIII:
 * radius r).
 *
 *   out = sorted union over i in anchor set of [max(0, i - r), min(t - 1, i + r)]
 *
 * anchor_idx[b,h,0:anchor_count) must be ascending and unique (as
 * prhs_select_topk writes it). radius 0 returns the anchor set unchanged.
 * out_cap must be >= min(t, (2r + 1) * anchor_cap). Counts are clamped to
 * [0, anchor_cap] and writes never pass out_cap.
 * Optional similarity gate (Fig. 8, Fig. 9(c)): when q_cur, q_anchor and
 * reuse_ok are all non-NULL, reuse_ok[b,h] = (cos(q_cur[b,h], q_anchor[b,h]) >=
 * sim_tau); the dilated set is written either way and the caller refreshes
 * the heads whose flag is 0. The queries use dims->dtype and layout [B,H_q,d].
 */
int prhs_cis_reuse(const prhs_dims* dims, const int32_t* anchor_idx, int32_t anchor_cap,
                   const int32_t* anchor_count, int32_t radius, const void* q_cur,
                   const void* q_anchor, float sim_tau, int32_t* out_idx, int32_t out_cap,
                   int32_t* out_count, int32_t* reuse_ok, hipStream_t stream);

/*
 * prhs_sparse_decode -- attention over the selected entries only (Abstract;
 * Table V caption), with the softmax renormalised over the set:
 *
 *   m_S = max_{i in S} s_i,  out = sum_{i in S} e^{s_i - m_S} v_i / sum_{i in S} e^{s_i - m_S}
 *   lse_sel = m_S + log sum_{i in S} e^{s_i - m_S}
 *
 * S = idx[b,h,0:count[b,h]). s_i is read from sel_scores when it is non-NULL
 * (fp32 [B, H_q, idx_cap] in idx order, as prhs_select_topk writes it), else
 * gathered from `scores` when that is non-NULL (the scores of the same step
 * from prhs_score); otherwise the K rows at S are gathered and scored (q and
 * k must then be non-NULL). With >= 128 (b, h) heads, or idx_cap <= 256, one
 * workgroup attends over a head's whole set (idx_cap <= 8192); otherwise the
 * set is split over workgroups and the partial (max, sum, output) triples are
 * merged exactly. Either way the result is the same up to the order of the
 * fp32 sums.
 * Indices outside [0, t) are skipped; counts are clamped to [0, idx_cap]; an
 * empty set gives out = 0, lse_sel = -inf.
 * Fused dropped mass: when lse_all and delta are non-NULL,
 * delta = clamp(-expm1(lse_sel - lse_all), 0, 1) and, if tau is non-NULL,
 * tau = 1 - delta.
 * ws: at least prhs_workspace_bytes(dims, PRHS_OP_DECODE, idx_cap) bytes.
 */
int prhs_sparse_decode(const prhs_dims* dims, const void* q, const void* k, const void* v,
                       const int32_t* idx, int32_t idx_cap, const int32_t* count,
                       const float* sel_scores, const float* scores, const float* lse_all,
                       float* out, float* lse_sel, float* delta, float* tau, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * prhs_sparse_decode_noalloc -- prhs_sparse_decode without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *
 * The operation, the arguments (all but ws and ws_bytes), the results and the
 * validation are those of prhs_sparse_decode. When the decode splits a head's
 * set over workgroups, the split partials go to a scratch array the library
 * keeps in device memory: one per GPU, PRHS_NOALLOC_SCRATCH_BYTES bytes, held
 * until the process ends (its address is looked up on the first call on each
 * device). The decode splits unless idx_cap <= 256, or idx_cap <= 8192 and
 * B * H_q >= 128 (then one workgroup per head needs no partials). A split
 * decode needs prhs_workspace_bytes(dims, PRHS_OP_DECODE, idx_cap) bytes; a call
 * that needs more than PRHS_NOALLOC_SCRATCH_BYTES returns PRHS_E_WORKSPACE with
 * nothing enqueued. The call allocates nothing. All calls on one GPU share its
 * scratch array, and each leaves its partials there: calls whose work
 * overlaps in time on one GPU (other streams, other threads) race on it and
 * must not be issued.
 */
#define PRHS_NOALLOC_SCRATCH_BYTES (4u << 20)

int prhs_sparse_decode_noalloc(const prhs_dims* dims, const void* q, const void* k, const void* v,
                               const int32_t* idx, int32_t idx_cap, const int32_t* count,
                               const float* sel_scores, const float* scores, const float* lse_all,
                               float* out, float* lse_sel, float* delta, float* tau,
                               hipStream_t stream);

/*
 * prhs_reuse_step -- one CIS reuse step in a single call: the dilation of
 * prhs_cis_reuse (without its similarity gate) followed by prhs_sparse_decode
 * over the dilated set, with K and V rows gathered (Fig. 4: the set of an
 * earlier query serves the next queries, grown around its clusters; Table
 * VIII: radius r).
 *
 * Results are those of the two calls in sequence, bit for bit: out_idx,
 * out_count, out and lse_sel. Argument rules are the union of the two calls'
 * rules; q, k and v are required. No dropped mass is formed, since a reuse
 * step has no dense log-sum-exp. When the heads fill the chip (or out_cap <=
 * 256), out_cap <= 8192 and 2r + 1 <= 64, one kernel per step does both.
 * ws: at least prhs_workspace_bytes(dims, PRHS_OP_DECODE, out_cap) bytes.
 */
int prhs_reuse_step(const prhs_dims* dims, const int32_t* anchor_idx, int32_t anchor_cap,
                    const int32_t* anchor_count, int32_t radius, const void* q, const void* k,
                    const void* v, int32_t* out_idx, int32_t out_cap, int32_t* out_count,
                    float* out, float* lse_sel, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * prhs_anchor_step -- one exact-retrieval decode step in a single call: the
 * score scan, the selection (TOPN or DELTA, as prhs_select_topk) and the
 * sparse decode with the fused dropped mass, enqueued back to back on
 * `stream` (Fig. 4: the query whose critical set is computed exactly; the
 * Abstract: selection ahead of attention with the dropped mass controlled).
 *
 * Results are those of the three calls in sequence: scores (but see theta
 * below), lse_all, idx, count, cap_hit (nullable), out, lse_sel, delta and
 * tau (nullable; tau needs delta). The dense log-sum-exp is merged inside the selection kernel
 * from the scan's per-chunk partials, so no separate merge runs. Argument
 * rules are the union of the three calls' rules.
 *
 * In either mode, with fp16 rows of head_dim 128 and n_budget (the TOPN
 * budget or the DELTA cap) <= 2048, each head's selection workgroup also
 * computes its attention: the selection is bit-identical to the three calls, and out,
 * lse_sel, delta and tau equal theirs up to the order of the fp32 sums.
 *
 * theta (nullable, fp32 [B, H_q], in/out; TOPN only): a per-head score
 * threshold hint, per unit query norm. The scan also hands the keys whose
 * score is >= theta * |q[b,h]| (fp32 Euclidean norm of the query row) to the
 * selection, which selects among them alone when they include the top
 * n_budget (at least n_budget of them and at most a few thousand) and
 * otherwise searches all keys, so the result never depends on the hint. NaN,
 * or a product theta * |q| that is not finite, means no hint. On return theta
 * holds a hint for the next step of the same heads: this step's boundary
 * score less a margin, divided by this step's |q| (adjacent decode queries
 * point in similar directions: Fig. 2, Fig. 10; their norms may differ:
 * Fig. 8). Initialise it to NaN.
 * With fp16 rows of head_dim 128 (and ctx_len * kv_stride_t * 2 < 2^32), a
 * head with a finite hint gets no scores row from the scan: its row is left
 * as it was, unless its hinted keys miss the answer, in which case the
 * selection recomputes the row (bit-identical to the scan's) before its full
 * search. Heads without a hint, and every other shape, get their rows.
 * ws: at least prhs_workspace_bytes(dims, PRHS_OP_ANCHOR_STEP, idx_cap) bytes.
 */
int prhs_anchor_step(const prhs_dims* dims, int32_t mode, int32_t n_budget, float delta_target,
                     const void* q, const void* k, const void* v, float* scores, float* lse_all,
                     int32_t* idx, int32_t idx_cap, int32_t* count, int32_t* cap_hit, float* out,
                     float* lse_sel, float* delta, float* tau, float* theta, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/*
 * prhs_dropped_mass -- dropped and retained attention mass of the selected
 * sets (Table I: delta(.), tau(.)):
 *   delta = clamp(-expm1(lse_sel - lse_all), 0, 1),  tau = 1 - delta.
 * tau may be NULL.
 */
int prhs_dropped_mass(const prhs_dims* dims, const float* lse_sel, const float* lse_all,
                      float* delta, float* tau, hipStream_t stream);

/*
 * prhs_adaptive_step -- one decode step of critical-index-set sharing with a
 * per-head similarity gate (Fig. 4: one query's set serves the next queries,
 * dilated; Fig. 8 and Fig. 9(c): sharing only while sim(q, q') >= tau;
 * Table VIII: block size s, threshold tau, radius r).
 *
 * Per head h, all on the device:
 *   refresh[h] = force_refresh || anchor_count[h] == 0
 *                || cos(q[h], anchor_q[h]) < sim_tau
 *   refresh heads: the exact top-n_budget over a fresh score scan (as
 *     prhs_anchor_step in TOPN mode) becomes the head's anchor set
 *     (anchor_idx, anchor_count), anchor_q[h] = q[h], attention runs over the
 *     new set, and lse_all, delta and tau are written;
 *   other heads: the anchor set dilated by `radius` (as prhs_cis_reuse) is
 *     written to dil_idx / dil_count and attention runs over it with gathered
 *     K and V rows; lse_all, delta and tau are left untouched (no scan ran).
 * A KV group with no refreshing head is not scanned. The caller passes
 * force_refresh = 1 on every s-th step (block size s); the gate then decides
 * the steps in between.
 * State, caller-owned and kept across steps: anchor_idx [B,H_q,n_budget],
 * anchor_count [B,H_q] (all zero before the first step), anchor_q [B,H_q,d]
 * (element type of q). Outputs: refresh [B,H_q] int32 0/1; sim (nullable)
 * fp32 [B,H_q], the cosine the gate used (NaN before a head's first anchor);
 * out, lse_sel; delta and tau (nullable; tau needs delta); theta (nullable)
 * as in prhs_anchor_step. Requires 1 <= n_budget <= t, radius >= 0,
 * dil_cap >= min(t, (2 radius + 1) n_budget), t <= PRHS_MAX_SELECT_CTX,
 * sim_tau not NaN.
 * ws: at least prhs_workspace_bytes(dims, PRHS_OP_ANCHOR_STEP, dil_cap) bytes.
 */
int prhs_adaptive_step(const prhs_dims* dims, int32_t n_budget, int32_t radius,
                       int32_t force_refresh, float sim_tau, const void* q, const void* k,
                       const void* v, float* scores, float* lse_all, int32_t* anchor_idx,
                       int32_t* anchor_count, void* anchor_q, int32_t* dil_idx, int32_t dil_cap,
                       int32_t* dil_count, int32_t* refresh, float* sim, float* out,
                       float* lse_sel, float* delta, float* tau, float* theta, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * prhs_random_expand -- the RandomExpansion control of Table VI (Panel A): the
 * anchor set grown to a matched size m with randomly chosen keys instead of
 * by dilation, for budget-matched comparisons with prhs_cis_reuse.
 *
 *   out = anchor set  U  the (m - |S_a|) keys outside it with the smallest
 *         draws[b,h,i] & 0x7FFFFF (the lower index on equal draws)
 *
 * draws: int32 [B, H_q, t] contiguous, caller-supplied random integers (only
 * the low 23 bits are used). anchor_idx [B,H_q,anchor_cap] ascending and
 * unique, anchor_count <= anchor_cap <= m <= t, out_cap >= m; out ascending,
 * out_count[b,h] = m. t <= PRHS_MAX_SELECT_CTX.
 * ws: at least prhs_workspace_bytes(dims, PRHS_OP_EXPAND, 0) bytes (a control
 * score row per head).
 */
int prhs_random_expand(const prhs_dims* dims, const int32_t* anchor_idx, int32_t anchor_cap,
                       const int32_t* anchor_count, const int32_t* draws, int32_t m,
                       int32_t* out_idx, int32_t out_cap, int32_t* out_count, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * prhs_dense_decode -- dense decode attention over all t keys: the baseline
 * the sparse path is compared with (Table IV: attention-operator latency
 * against dense FlashAttention; Abstract: speedup over the dense baseline).
 *
 *   out[b,h,:]  = sum_i softmax_i(s[b,h,:]) * V[b,h/G,i,:],  s as in prhs_score
 *   lse[b,h]    = log sum_i exp(s[b,h,i])   (the dense log-sum-exp)
 *
 * One pass: K and V are each read once, split over keys; the per-split
 * (max, sum, output) partials are merged exactly. No scores are written.
 * q, k, v, out, lse and ws are required; q, k, v 16-byte aligned.
 * ws: at least prhs_workspace_bytes(dims, PRHS_OP_DENSE, 0) bytes.
 */
int prhs_dense_decode(const prhs_dims* dims, const void* q, const void* k, const void* v,
                      float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * prhs_append_kv -- append one decode step's key and value rows to the cache
 * (Table I: t counts the decode steps, so the cache gains one row per step):
 * for every b < batch and g < n_kv_heads
 *   k[b, g, pos, :] = k_new[b, g, :],   v[b, g, pos, :] = v_new[b, g, :]
 * k and v are laid out as dims describes (kv_stride_*, d contiguous, shared by
 * k and v); k_new and v_new are contiguous [batch, n_kv_heads, head_dim] in
 * dims->dtype. pos must lie in [0, ctx_len) (grow ctx_len to t, then append
 * at pos = t - 1); the caller guarantees that row pos exists in its
 * allocation. Every pointer is required and 16-byte aligned.
 */
int prhs_append_kv(const prhs_dims* dims, const void* k_new, const void* v_new, void* k, void* v,
                   int32_t pos, hipStream_t stream);

/* Workspace bytes needed by `op` (PRHS_OP_*) for these dims; `cap` is the
 * idx_cap of prhs_sparse_decode / prhs_anchor_step and is ignored otherwise.
 * Returns 0 for invalid dims. */
size_t prhs_workspace_bytes(const prhs_dims* dims, int32_t op, int32_t cap);

/* Static text for a status code. */
const char* prhs_status_string(int status);

/* Thread-local detail of the last error returned on this thread ("" if none). */
const char* prhs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PRHS_H */
