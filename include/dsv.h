/*
 * dsv.h — C ABI of the DSV dynamic-sparsity attention hot path on MI355X (gfx950).
 *
 * The operations follow the technical summaries of
 *   "DSV: Exploiting Dynamic Sparsity to Accelerate Large-Scale Video DiT Training"
 *   (gist.science/{zh,pt,fr,ko}/paper/2502.07590):
 *   - zh §2.1 "Two-Stage Training Algorithm" / pt §2A / fr §2A / ko §2가: per-head low-rank
 *     factors approximate QK^T and are used to estimate the critical KV pairs; full attention
 *     is then computed on the critical pairs only.
 *   - zh §2.2 "Efficient Kernels" / pt §2B / fr §2B / ko §2나: the low-rank MatMul and the
 *     top-k are fused so the S x S score matrix is never stored (memory O(S^2) -> O(S*k));
 *     spatio-temporally adjacent queries are grouped and share one list of critical KV indices.
 *
 * Conventions shared by every entry point
 *   Token grid: a sample is a latent video of T x Hh x W tokens, flattened row-major,
 *     token n = (t*Hh + y)*W + x, S = T*Hh*W.
 *   Query groups: gt x gh x gw blocks of adjacent tokens (gt | T, gh | Hh, gw | W).
 *     G = gt*gh*gw queries per group, NG = S/G groups per (batch, head). Group index
 *     g = (a*(Hh/gh) + b)*(W/gw) + c for block (a,b,c); its members are enumerated
 *     row-major over (dt,dy,dx). Groups never cross samples.
 *   Tensors Q, K, V, O, dO, dQ, dK, dV: [B][H][S][d] contiguous. LSE: [B][H][S] fp32.
 *     Q_lr, K_lr: [B][H][S][r] contiguous, same storage dtype as Q.
 *   idx (critical-KV lists), packed int32, no padding:
 *     row of (b,h,g) starts at NG*(b*sum_h k_h + sum_{h'<h} k_h') + g*k_h and holds k_h
 *     strictly ascending key indices in [0,S). Total length B*NG*sum_h k_h.
 *     A list that breaks this is memory-safe: the attention kernels clamp every key into
 *     [0,S) (a key >= S, and a negative one, is read as key S-1); the forward and dQ then
 *     use the clamped keys as listed (repeats counted), and dK/dV are unspecified (finite)
 *     for such a list.
 *   k_per_head: HOST array of H int32, 1 <= k_h <= S (k_h = S is dense attention).
 *   Scale: softmax(scale * q.k), no causal mask; the LSE is natural-log and includes the scale.
 *
 * Ownership and concurrency
 *   The caller owns every buffer. Every pointer except k_per_head and the problem
 *   descriptor is a device pointer. The library allocates nothing and keeps no state:
 *   calls are re-entrant and thread-safe. `stream` is a hipStream_t (NULL = legacy default
 *   stream). Calls are asynchronous: inputs must stay unchanged, and outputs unread, until
 *   the stream has passed the call. Outputs are overwritten, never accumulated. A
 *   workspace belongs to one call at a time: calls in flight together need separate ones.
 *
 * Errors
 *   Arguments are validated before anything is enqueued. On a non-OK status nothing has been
 *   enqueued and the outputs are untouched. DSV_ERR_HIP reports a failed launch; device faults
 *   surface at the caller's next synchronisation. dsv_last_error() returns a thread-local
 *   message describing the last non-OK status.
 */
#ifndef DSV_H_
#define DSV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DSV_FP32 = 0, DSV_BF16 = 1 } dsv_dtype;

/* How the per-query low-rank scores of a group are combined into one group score.
 * SUM: sigma[g][m] = sum_{n in g} Q_lr[n].K_lr[m] (MEAN ranks identically).
 * MAX: sigma[g][m] = max_{n in g} Q_lr[n].K_lr[m] (the per-query S x S scores, never stored;
 * about G times the MFMA work of SUM per pass over the keys). */
typedef enum { DSV_GROUP_SUM = 0, DSV_GROUP_MAX = 1 } dsv_reduce;

typedef enum {
  DSV_OK = 0,
  DSV_ERR_NULL = 1,        /* a required pointer is NULL */
  DSV_ERR_SHAPE = 2,       /* non-positive size, group extents do not divide the grid, ... */
  DSV_ERR_K = 3,           /* some k_h outside [1, S] */
  DSV_ERR_DTYPE = 4,       /* dtype not one of dsv_dtype */
  DSV_ERR_ALIGN = 5,       /* a device pointer is not 16-byte aligned */
  DSV_ERR_WORKSPACE = 6,   /* ws_bytes < dsv_workspace_bytes(...) */
  DSV_ERR_UNSUPPORTED = 7, /* a valid but unimplemented case (head_dim, rank, G, reduce) */
  DSV_ERR_HIP = 8          /* the HIP runtime reported an error at launch */
} dsv_status;

typedef enum { DSV_OP_TOPK = 0, DSV_OP_FWD = 1, DSV_OP_BWD = 2 } dsv_op;

typedef struct {
  int32_t batch, heads;          /* B, H */
  int32_t frames, height, width; /* T, Hh, W */
  int32_t head_dim, rank;        /* d in {64,128}; r in {16,32,48,64} */
  int32_t gt, gh, gw;            /* group extents; G = gt*gh*gw must be 16, 32, 48 or 64 */
  int32_t dtype;                 /* dsv_dtype of Q,K,V,O,dO,Q_lr,K_lr */
} dsv_problem;

/* Minimum bytes of device workspace `op` needs for this problem. DSV_OP_TOPK and DSV_OP_FWD
 * need none (their ws may be NULL). DSV_OP_BWD on the bf16 path needs the per-edge dV|dK
 * staging rows of one (b,h) head (about NG*k32*(4*d + 4.5) bytes, k32 = max k rounded up
 * to a multiple of 32, plus small per-bucket tables); a
 * larger workspace lets one launch cover several heads. The fp32 path needs 16*B*H*S*d bytes
 * (fixed-point dV and dK accumulators). Returns (size_t)-1 if the problem is invalid. */
size_t dsv_workspace_bytes(int op, const dsv_problem* p, const int32_t* k_per_head);

/* Total int32 elements of the packed idx array: B * NG * sum_h k_h (0 if invalid). */
int64_t dsv_idx_elems(const dsv_problem* p, const int32_t* k_per_head);

/* Element offset of row (b,h,g) inside the packed idx array (-1 if out of range). */
int64_t dsv_idx_row_offset(const dsv_problem* p, const int32_t* k_per_head, int32_t b,
                           int32_t h, int32_t g);

/* Critical-KV estimation: fused low-rank group scoring + exact per-group top-k.
 * (DSV summaries: zh §2.1 and §2.2, pt §2A-§2B, fr §2A-§2B, ko §2가-§2나.)
 *   q_lr, k_lr : [B][H][S][r] device, dtype p->dtype.
 *   k_per_head : host [H].
 *   reduce     : DSV_GROUP_SUM or DSV_GROUP_MAX.
 *   idx        : device int32, dsv_idx_elems() elements, written.
 * For every (b,h,g): with SUM, sigma[m] = (sum_{n in g} q_lr[n]) . k_lr[m] evaluated in fp32
 * (equal to summing the per-query scores, by linearity); with MAX, sigma[m] = the largest
 * per-query score q_lr[n] . k_lr[m] over the members (fp32). The row holds the k_h keys with
 * the largest sigma, equal scores ranked by lower key index, written in ascending key order.
 * Exactness: the scores, hence idx, are exact when Q_lr and K_lr hold integers with
 * G*max|q| < 2^16 and G*r*max|q|*max|k| < 2^24 (SUM: the bf16 path splits the group sum into
 * two bf16 terms; outside this domain the group sum is rounded to 16 significant bits; MAX:
 * r*max|q|*max|k| < 2^24). The S x S score matrix is never stored.
 *   ws, ws_bytes : optional device workspace (may be NULL / 0; SUM ignores it). With MAX and
 *                  ws 256-byte aligned, ws_bytes >= c * dsv_topk_max_cache_bytes(p) (c >= 1)
 *                  lets c (b,h) slots per launch keep their NG x S group scores in ws between
 *                  the passes of the selection instead of recomputing the member products in
 *                  every pass; the result is the same. Contents on entry ignored, clobbered.
 * The stream gets one launch, or with the MAX cache one launch per c slots. */
int dsv_lowrank_topk(const dsv_problem* p, const void* q_lr, const void* k_lr,
                     const int32_t* k_per_head, int reduce, int32_t* idx, void* ws,
                     size_t ws_bytes, void* stream);

/* Workspace bytes per (b,h) slot for the MAX score cache of dsv_lowrank_topk: NG rows of
 * S keys rounded up to a multiple of 128, 4 bytes each, the total rounded up to 256
 * ((size_t)-1 if the problem is invalid). */
size_t dsv_topk_max_cache_bytes(const dsv_problem* p);

/* Adaptive k: the number of keys per group that carry a given share of the group's estimated
 * attention mass. (DSV summaries: zh §2.1 stage two, "critical KV estimation": the low-rank
 * estimate of QK^T identifies the KV pairs that contribute more than 90% of the attention
 * score; pt §2A, fr §2A, ko §2가.)
 *   q_lr, k_lr  : as for dsv_lowrank_topk (group scores sigma[g][m], SUM reduction).
 *   logit_scale : > 0 and finite; the estimated logit of key m for group g is
 *                 logit_scale * sigma[g][m] (scale / G makes it the mean of the members'
 *                 scaled low-rank logits).
 *   mass        : in (0, 1], e.g. 0.9.
 *   k_group     : device int32 [B][H][NG] or NULL, written: k of every group.
 *   k_head      : device int32 [H], written: the largest k of the head's groups over the batch.
 * A group's k is the smallest number of its keys whose softmax weights
 * w_m = exp(logit_scale * (sigma[g][m] - max_m' sigma[g][m'])), largest first, reach `mass` of
 * the row's total weight. The largest weights belong to the largest scores, so the first k
 * keys of dsv_lowrank_topk (same scores, same order) carry that share; with k_per_head =
 * k_head every group of the head gets at least its own k keys.
 * Arithmetic: each w_m is evaluated in fp64 and rounded to an integer multiple of 2^-P,
 * P = 62 - (bit length of S); all sums are exact integer sums, so the result does not depend
 * on the order of the work and repeats bit for bit. Compared with exact arithmetic, each
 * prefix sum of the weights and the target mass * total are off by at most S * 2^-(P+1) +
 * 2^-P plus a few fp64 roundings of the total: k can differ from the exact rule only in a row
 * where some prefix sum lies that close to mass * total. Launches on `stream`; no workspace. */
int dsv_adaptive_k(const dsv_problem* p, const void* q_lr, const void* k_lr, float logit_scale,
                   double mass, int32_t* k_group, int32_t* k_head, void* stream);

/* Query-grouped sparse attention, forward.
 * (DSV summaries: zh §2.1 "sparse computation" bullet and §2.2 "Query Grouping".)
 *   q,k,v : [B][H][S][d] device, dtype p->dtype.   idx, k_per_head: as above.
 *   o     : [B][H][S][d] device, dtype p->dtype (written).
 *   lse   : [B][H][S] fp32 device (written): log sum_m exp(scale*q.k_m) over the row's keys.
 *   scale : > 0 and finite (DSV_ERR_SHAPE otherwise), e.g. 1/sqrt(d).
 * For query n in group g: O[n] = sum_{m in idx(g)} softmax_m(scale*q_n.k_m) v_m, computed with
 * fp32 accumulation (bf16 MFMA operands on the bf16 path). */
int dsv_sparse_attn_fwd(const dsv_problem* p, const void* q, const void* k, const void* v,
                        const int32_t* idx, const int32_t* k_per_head, float scale, void* o,
                        float* lse, void* ws, size_t ws_bytes, void* stream);

/* Query-grouped sparse attention, backward (idx is a constant: no gradient flows to the
 * low-rank factors).
 *   o, d_o : [B][H][S][d] device, dtype p->dtype (o is the forward output).
 *   lse    : forward LSE.   scale: as for the forward (> 0 and finite).
 *   dq,dk,dv : [B][H][S][d] fp32 device (written in full: every key receives the sum over
 *              all groups that selected it, 0 if none did).
 *   ws       : device, 256-byte aligned, at least dsv_workspace_bytes(DSV_OP_BWD, ...) bytes
 *              (bf16 path); owned by the caller, contents on entry ignored, clobbered.
 * With P = exp(scale*q.k - LSE), Delta_n = dO_n.O_n, dS = P*(dO.v - Delta):
 *   dQ_n = scale*sum_m dS[n,m] k_m,  dK_m = scale*sum_n dS[n,m] q_n,  dV_m = sum_n P[n,m] dO_n.
 * bf16 path: each (group, selected key) edge writes its partial dV and dK rows to its own
 * staging row in ws, with one scale per (tensor, group, 16-key block) taken from the block's
 * largest entry m (for dK after the softmax scale): 8-bit codes when d = 128 and m <= 0.125
 * (absolute error <= m/254 per entry), else fp16 scaled by a power of two (relative error
 * <= 2^-11 per entry); a second kernel sums each 32-key bucket's rows in a fixed order.
 * dK/dV are therefore bitwise reproducible from run to run. fp32 path: each group's partial
 * dV and dK sums are rounded to multiples of 2^-32 and added as 64-bit integers in ws, then
 * converted (error <= 2^-33 per group's contribution; reproducible bit for bit; |sums| < 2^31).
 * The stream is used for several launches per call (heads are processed in chunks that fit
 * ws). Unsupported (DSV_ERR_UNSUPPORTED) when NG * k32 >= 2^27 staging rows per head. */
int dsv_sparse_attn_bwd(const dsv_problem* p, const void* q, const void* k, const void* v,
                        const void* o, const void* d_o, const float* lse, const int32_t* idx,
                        const int32_t* k_per_head, float scale, float* dq, float* dk, float* dv,
                        void* ws, size_t ws_bytes, void* stream);

/* Size of the fixed device scratch array of dsv_sparse_attn_bwd_noalloc: 256 MiB per GPU,
 * held from the library's load until the process ends. */
#define DSV_NOALLOC_SCRATCH_BYTES (256u * 1024u * 1024u)

/* dsv_sparse_attn_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). It runs the same kernels with a fixed scratch array of
 * DSV_NOALLOC_SCRATCH_BYTES that the library keeps on each GPU, and calls no allocator.
 *   Arguments, layouts, results and errors: as dsv_sparse_attn_bwd (the results are the same
 *   bits). stream must belong to the calling thread's current device.
 *   DSV_ERR_WORKSPACE (nothing enqueued) when dsv_workspace_bytes(DSV_OP_BWD, p, k_per_head)
 *   exceeds DSV_NOALLOC_SCRATCH_BYTES: the heaviest head's staging rows must fit (S = 16K,
 *   d = 64, G = 64, k = 10% needs about 112 MB; S = 64K, d = 128, k = 10% does not fit).
 *   DSV_ERR_HIP if the scratch array's address cannot be looked up.
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's contents: calls
 * that overlap on one GPU (several streams or threads) race, and must be serialised by the
 * caller. The first call on each device looks the array's address up (no allocation). */
int dsv_sparse_attn_bwd_noalloc(const dsv_problem* p, const void* q, const void* k,
                                const void* v, const void* o, const void* d_o, const float* lse,
                                const int32_t* idx, const int32_t* k_per_head, float scale,
                                float* dq, float* dk, float* dv, void* stream);

/* Number of head chunks dsv_sparse_attn_bwd uses with a workspace of ws_bytes: the heads
 * are processed in that many groups of launches, each staging its rows in the workspace.
 * 1 on the fp32 path; -1 if the problem is invalid or ws_bytes is below the minimum. */
int dsv_bwd_chunks(const dsv_problem* p, const int32_t* k_per_head, size_t ws_bytes);

/* dsv_sparse_attn_bwd for profiling (bf16 path only): identical work and results, and it
 * also records caller-created hipEvent_t handles on `stream` around the stages of every head
 * chunk c: events[4c] before the chunk's index pre-passes, events[4c+1] before its backward
 * kernel, events[4c+2] before its bucket reduce, events[4c+3] after it. n_events must equal
 * 4 * dsv_bwd_chunks(p, k_per_head, ws_bytes); the caller owns the events (created with
 * timing enabled) and reads them after the stream has passed the call. */
int dsv_sparse_attn_bwd_profiled(const dsv_problem* p, const void* q, const void* k,
                                 const void* v, const void* o, const void* d_o, const float* lse,
                                 const int32_t* idx, const int32_t* k_per_head, float scale,
                                 float* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                                 void* stream, void* const* events, int n_events);

/* ---- Planning (host only; no HIP call, nothing enqueued) ---------------------------------- */

/* Head placement over n_parts devices (DSV summaries: zh §2.3 "Head-wise CP Re-balancing",
 * pt §2C, fr §2C, ko §2다: heads are assigned to GPUs by their sparsity so the compute load
 * balances; db-SP summary, "核心方法" (core method): a head-level greedy, and the sparse
 * imbalance ratio rho_s = max load / mean load from its "关键观察" (key observations)).
 *   k_per_head   : host [heads], each >= 1.
 *   fixed_cost, cost_per_k : cost of head h = fixed_cost + cost_per_k * k_h (any unit, >= 0,
 *                  not both 0), e.g. the estimator's time per head and the attention time per
 *                  unit of k (dsv_default_cost_model gives measured MI355X figures).
 *   part_of_head : host [heads], written: the part (0 .. n_parts-1) each head goes to.
 *   part_load    : host [n_parts] or NULL, written: the summed cost of each part.
 *   rho          : host or NULL, written: max part load / mean part load (>= 1).
 * Longest-processing-time greedy: heads in decreasing cost (equal costs: lower head index
 * first), each to the part with the least load so far (equal loads: lower part index). The
 * largest load is at most (4/3 - 1/(3 n_parts)) times the optimum. The kernels launch the heads
 * of one device in this same decreasing-cost order. */
int dsv_plan_heads(const int32_t* k_per_head, int32_t heads, int32_t n_parts, double fixed_cost,
                   double cost_per_k, int32_t* part_of_head, double* part_load, double* rho);

/* The planner's processing order: heads by decreasing cost fixed_cost + cost_per_k * k_h
 * (equal costs: lower head index first), i.e. the order in which dsv_plan_heads places them.
 * On one device (n_parts = 1) every head lands on it in this order, and the kernels launch the
 * heads of a problem in the order dsv_plan_order(k_per_head, H, 0, 1, order) gives.
 * (DSV summaries zh §2.3 head re-balancing; db-SP summary, head-level greedy.)
 *   order : host [heads], written: head indices, first processed first. */
int dsv_plan_order(const int32_t* k_per_head, int32_t heads, double fixed_cost,
                   double cost_per_k, int32_t* order);

/* Per-unit costs of this library's kernels on one MI355X, for planning and dispatch. */
typedef struct {
  double topk_ns_per_score;  /* critical-KV estimation, per (group, key) score */
  double attn_ns_per_edge;   /* sparse attention, per (group, selected key) edge */
} dsv_cost_model;

/* Fills `cm` with figures measured on MI355X (the S=64K workload, scaled to the problem's
 * rank, head_dim and group size in proportion to the work per unit): forward only
 * (with_backward = 0) or forward + backward (1). */
int dsv_default_cost_model(const dsv_problem* p, int with_backward, dsv_cost_model* cm);

/* Dense-versus-sparse choice per head (DSV summaries: zh §2.1 stage two, the OP Dispatcher
 * decides per block from its sparsity whether sparse attention runs). Per (b, h) the sparse
 * path costs NG*S*topk_ns_per_score + NG*k_h*attn_ns_per_edge and dense attention
 * NG*S*attn_ns_per_edge; a head goes dense when that is not more, i.e. when
 * k_h >= S * (1 - topk_ns_per_score / attn_ns_per_edge).
 *   k_in      : host [heads], the sparse k_h.
 *   k_out     : host [heads], written: S for a dense head, else k_in[h]. Dense heads run
 *               through the same kernels (dsv_lowrank_topk writes the full ascending row for
 *               k_h = S without scoring).
 *   n_dense   : host or NULL, written: the number of dense heads. */
int dsv_dispatch_k(const dsv_problem* p, const int32_t* k_in, const dsv_cost_model* cm,
                   int32_t* k_out, int32_t* n_dense);

/* Validation only: returns the status the corresponding call would return for these
 * arguments before enqueueing anything (no HIP call is made). Pointers are checked for NULL
 * and 16-byte alignment; pass any non-NULL aligned values to check shapes alone. */
int dsv_validate(int op, const dsv_problem* p, const int32_t* k_per_head, int reduce,
                 const void* const* ptrs, int n_ptrs, size_t ws_bytes);

const char* dsv_status_string(int status);
const char* dsv_last_error(void);

/* Library version, "major.minor.patch". */
const char* dsv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSV_H_ */
