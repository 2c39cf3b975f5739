// dsv_api.cpp — the C ABI: argument validation (no HIP calls) and dispatch to the launchers.
//
// Every check runs before anything is enqueued, so a non-OK status leaves the stream and the
// outputs untouched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "dsv_internal.h"

namespace dsv {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

static int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int validate_problem(const dsv_problem* p, const int32_t* kph, Geom* geo) {
  if (!p) return fail(DSV_ERR_NULL, "problem descriptor is NULL");
  if (!kph) return fail(DSV_ERR_NULL, "k_per_head is NULL");
  const int vals[] = {p->batch, p->heads, p->frames, p->height, p->width,
                      p->head_dim, p->rank, p->gt, p->gh, p->gw};
  for (int v : vals)
    if (v <= 0) return fail(DSV_ERR_SHAPE, "every size in the problem must be positive");
  if (p->dtype != DSV_FP32 && p->dtype != DSV_BF16)
    return fail(DSV_ERR_DTYPE, "dtype %d is not DSV_FP32 or DSV_BF16", p->dtype);
  if (p->frames % p->gt || p->height % p->gh || p->width % p->gw)
    return fail(DSV_ERR_SHAPE, "group %dx%dx%d does not divide the %dx%dx%d token grid", p->gt,
                p->gh, p->gw, p->frames, p->height, p->width);
  const long long S = (long long)p->frames * p->height * p->width;
  if (S > (1LL << 24))
    return fail(DSV_ERR_UNSUPPORTED, "S = %lld tokens exceeds 2^24", S);
  if (p->heads > kMaxHeads)
    return fail(DSV_ERR_UNSUPPORTED, "heads = %d exceeds %d", p->heads, kMaxHeads);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(DSV_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", p->head_dim);
  if (p->rank % 16 || p->rank > 64)
    return fail(DSV_ERR_UNSUPPORTED, "rank %d (supported: 16, 32, 48, 64)", p->rank);
  const int G = p->gt * p->gh * p->gw;
  if (G % 16 || G > 64)
    return fail(DSV_ERR_UNSUPPORTED, "group size %d (supported: 16, 32, 48, 64)", G);
  long long ksum = 0;
  for (int h = 0; h < p->heads; ++h) {
    if (kph[h] < 1 || kph[h] > S)
      return fail(DSV_ERR_K, "k_per_head[%d] = %d is outside [1, %lld]", h, kph[h], S);
    ksum += kph[h];
  }
  if (geo) {
    Geom& g = *geo;
    memset(&g, 0, sizeof(g));
    g.B = p->batch; g.H = p->heads; g.T = p->frames; g.Hh = p->height; g.W = p->width;
    g.S = (int)S; g.d = p->head_dim; g.r = p->rank; g.gt = p->gt; g.gh = p->gh; g.gw = p->gw;
    g.G = G; g.NG = (int)(S / G); g.nbh = p->height / p->gh; g.nbw = p->width / p->gw;
    g.dtype = p->dtype;
    g.ksum = ksum;
    long long acc = 0;
    for (int h = 0; h < p->heads; ++h) {
      g.k[h] = kph[h];
      g.pre[h] = acc;
      acc += kph[h];
    }
    // heads launch in the planner's order for a single device: the attention's cost per
    // head grows with k_h, so heavy heads go first (longest processing time first)
    double cost[kMaxHeads];
    for (int h = 0; h < p->heads; ++h) cost[h] = (double)kph[h];
    lpt_order(cost, p->heads, g.order);
  }
  return DSV_OK;
}

static int check_ptr(const void* ptr, const char* name, size_t align) {
  if (!ptr) return fail(DSV_ERR_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % align)
    return fail(DSV_ERR_ALIGN, "%s is not %zu-byte aligned", name, align);
  return DSV_OK;
}

// The kernels keep the running maximum on raw scores q.k, which orders logits only for a
// positive scale.
static int check_scale(float scale) {
  if (!(scale > 0.0f) || !isfinite(scale))
    return fail(DSV_ERR_SHAPE, "scale = %g: it must be positive and finite", (double)scale);
  return DSV_OK;
}

}  // namespace dsv

using namespace dsv;

extern "C" {

const char* dsv_version(void) { return "0.1.0"; }

const char* dsv_status_string(int s) {
  switch (s) {
    case DSV_OK: return "DSV_OK";
    case DSV_ERR_NULL: return "DSV_ERR_NULL";
    case DSV_ERR_SHAPE: return "DSV_ERR_SHAPE";
    case DSV_ERR_K: return "DSV_ERR_K";
    case DSV_ERR_DTYPE: return "DSV_ERR_DTYPE";
    case DSV_ERR_ALIGN: return "DSV_ERR_ALIGN";
    case DSV_ERR_WORKSPACE: return "DSV_ERR_WORKSPACE";
    case DSV_ERR_UNSUPPORTED: return "DSV_ERR_UNSUPPORTED";
    case DSV_ERR_HIP: return "DSV_ERR_HIP";
    default: return "DSV_ERR_UNKNOWN";
  }
}

const char* dsv_last_error(void) { return g_err; }

size_t dsv_workspace_bytes(int op, const dsv_problem* p, const int32_t* k_per_head) {
  if (op < DSV_OP_TOPK || op > DSV_OP_BWD) return (size_t)-1;
  Geom geo;
  if (validate_problem(p, k_per_head, &geo) != DSV_OK) return (size_t)-1;
  return op == DSV_OP_BWD ? bwd_workspace_bytes(geo) : 0;
}

int64_t dsv_idx_elems(const dsv_problem* p, const int32_t* k_per_head) {
  Geom g;
  if (validate_problem(p, k_per_head, &g) != DSV_OK) return 0;
  return (int64_t)g.B * g.NG * g.ksum;
}

int64_t dsv_idx_row_offset(const dsv_problem* p, const int32_t* k_per_head, int32_t b, int32_t h,
                           int32_t g) {
  Geom geo;
  if (validate_problem(p, k_per_head, &geo) != DSV_OK) return -1;
  if (b < 0 || b >= geo.B || h < 0 || h >= geo.H || g < 0 || g >= geo.NG) return -1;
  return geo.row_offset(b, h, g);
}

int dsv_validate(int op, const dsv_problem* p, const int32_t* k_per_head, int reduce,
                 const void* const* ptrs, int n_ptrs, size_t ws_bytes) {
  Geom geo;
  int st = validate_problem(p, k_per_head, &geo);
  if (st != DSV_OK) return st;
  static const char* topk_names[] = {"q_lr", "k_lr", "idx"};
  static const size_t topk_align[] = {16, 16, 4};
  static const char* fwd_names[] = {"q", "k", "v", "idx", "o", "lse"};
  static const size_t fwd_align[] = {16, 16, 16, 4, 16, 4};
  static const char* bwd_names[] = {"q", "k", "v", "o", "d_o", "lse", "idx", "dq", "dk", "dv"};
  static const size_t bwd_align[] = {16, 16, 16, 16, 16, 4, 4, 16, 16, 16};
  const char* const* names;
  const size_t* aligns;
  int n;
  switch (op) {
    case DSV_OP_TOPK:
      if (reduce != DSV_GROUP_SUM && reduce != DSV_GROUP_MAX)
        return fail(DSV_ERR_UNSUPPORTED, "unknown reduce %d", reduce);
      names = topk_names; aligns = topk_align; n = 3; break;
    case DSV_OP_FWD: names = fwd_names; aligns = fwd_align; n = 6; break;
    case DSV_OP_BWD: names = bwd_names; aligns = bwd_align; n = 10; break;
    default: return fail(DSV_ERR_UNSUPPORTED, "unknown op %d", op);
  }
  if (!ptrs || n_ptrs != n) return fail(DSV_ERR_NULL, "op %d expects %d pointers", op, n);
  for (int i = 0; i < n; ++i)
    if ((st = check_ptr(ptrs[i], names[i], aligns[i])) != DSV_OK) return st;
  if (op == DSV_OP_BWD && geo.dtype == DSV_BF16) {
    int kmax = 0;
    for (int h = 0; h < geo.H; ++h) kmax = std::max(kmax, geo.k[h]);
    const long long rows = (long long)geo.NG * ((kmax + 31) & ~31);
    if (rows >= (1LL << 27))
      return fail(DSV_ERR_UNSUPPORTED, "backward: %lld staging rows per head exceed 2^27", rows);
  }
  const size_t need = op == DSV_OP_BWD ? bwd_workspace_bytes(geo) : 0;
  if (ws_bytes < need)
    return fail(DSV_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, need);
  return DSV_OK;
}

int dsv_lowrank_topk(const dsv_problem* p, const void* q_lr, const void* k_lr,
                     const int32_t* k_per_head, int reduce, int32_t* idx, void* ws,
                     size_t ws_bytes, void* stream) {
  const void* ptrs[] = {q_lr, k_lr, idx};
  int st = dsv_validate(DSV_OP_TOPK, p, k_per_head, reduce, ptrs, 3, ws_bytes);
  if (st != DSV_OK) return st;
  Geom geo;
  validate_problem(p, k_per_head, &geo);
  int e = launch_topk(geo, q_lr, k_lr, reduce, idx, ws, ws ? ws_bytes : 0, stream);
  if (e) return fail(DSV_ERR_HIP, "top-k launch failed (hipError %d)", e);
  return DSV_OK;
}

size_t dsv_topk_max_cache_bytes(const dsv_problem* p) {
  std::vector<int32_t> ones(p && p->heads > 0 ? p->heads : 1, 1);
  Geom geo;
  if (validate_problem(p, ones.data(), &geo) != DSV_OK) return (size_t)-1;
  return topk_max_cache_slot_bytes(geo);
}

int dsv_adaptive_k(const dsv_problem* p, const void* q_lr, const void* k_lr, float logit_scale,
                   double mass, int32_t* k_group, int32_t* k_head, void* stream) {
  std::vector<int32_t> ones(p && p->heads > 0 ? p->heads : 1, 1);
  Geom geo;
  int st = validate_problem(p, ones.data(), &geo);
  if (st != DSV_OK) return st;
  if ((st = check_ptr(q_lr, "q_lr", 16)) || (st = check_ptr(k_lr, "k_lr", 16)) ||
      (st = check_ptr(k_head, "k_head", 4)))
    return st;
  if (k_group && reinterpret_cast<uintptr_t>(k_group) % 4)
    return fail(DSV_ERR_ALIGN, "k_group is not 4-byte aligned");
  if (!(logit_scale > 0.0f) || !isfinite(logit_scale))
    return fail(DSV_ERR_SHAPE, "logit_scale must be positive and finite");
  if (!(mass > 0.0 && mass <= 1.0)) return fail(DSV_ERR_SHAPE, "mass must be in (0, 1]");
  AdaptiveParams ap;
  ap.ls = (double)logit_scale;
  ap.fx = ldexp(1.0, adaptive_fx_bits(geo.S));
  ap.mass = mass;
  const int e = launch_adaptive_k(geo, q_lr, k_lr, ap, k_group, k_head, stream);
  if (e) return fail(DSV_ERR_HIP, "adaptive-k launch failed (hipError %d)", e);
  return DSV_OK;
}

int dsv_sparse_attn_fwd(const dsv_problem* p, const void* q, const void* k, const void* v,
                        const int32_t* idx, const int32_t* k_per_head, float scale, void* o,
                        float* lse, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  const void* ptrs[] = {q, k, v, idx, o, lse};
  int st = dsv_validate(DSV_OP_FWD, p, k_per_head, DSV_GROUP_SUM, ptrs, 6, ws_bytes);
  if (st != DSV_OK) return st;
  if ((st = check_scale(scale)) != DSV_OK) return st;
  Geom geo;
  validate_problem(p, k_per_head, &geo);
  int e = launch_attn_fwd(geo, q, k, v, idx, scale, o, lse, stream);
  if (e) return fail(DSV_ERR_HIP, "forward launch failed (hipError %d)", e);
  return DSV_OK;
}

static int bwd_common(const dsv_problem* p, const void* q, const void* k, const void* v,
                      const void* o, const void* d_o, const float* lse, const int32_t* idx,
                      const int32_t* k_per_head, float scale, float* dq, float* dk, float* dv,
                      void* ws, size_t ws_bytes, void* stream, void* const* events,
                      int n_events) {
  const void* ptrs[] = {q, k, v, o, d_o, lse, idx, dq, dk, dv};
  int st = dsv_validate(DSV_OP_BWD, p, k_per_head, DSV_GROUP_SUM, ptrs, 10, ws_bytes);
  if (st != DSV_OK) return st;
  if ((st = check_scale(scale)) != DSV_OK) return st;
  Geom geo;
  validate_problem(p, k_per_head, &geo);
  if (bwd_workspace_bytes(geo) > 0 && (st = check_ptr(ws, "ws", 256)) != DSV_OK) return st;
  if (events) {
    if (geo.dtype != DSV_BF16)
      return fail(DSV_ERR_UNSUPPORTED, "stage events are recorded on the bf16 path only");
    const int need = 4 * bwd_chunk_count(geo, ws_bytes);
    if (n_events != need)
      return fail(DSV_ERR_NULL, "expected %d stage events (4 per head chunk), got %d", need,
                  n_events);
    for (int i = 0; i < n_events; ++i)
      if (!events[i]) return fail(DSV_ERR_NULL, "stage event %d is NULL", i);
  }
  int e = launch_attn_bwd(geo, q, k, v, o, d_o, lse, idx, scale, dq, dk, dv, ws, ws_bytes,
                          stream, events);
  if (e) return fail(DSV_ERR_HIP, "backward launch failed (hipError %d)", e);
  return DSV_OK;
}

int dsv_sparse_attn_bwd(const dsv_problem* p, const void* q, const void* k, const void* v,
                        const void* o, const void* d_o, const float* lse, const int32_t* idx,
                        const int32_t* k_per_head, float scale, float* dq, float* dk, float* dv,
                        void* ws, size_t ws_bytes, void* stream) {
  return bwd_common(p, q, k, v, o, d_o, lse, idx, k_per_head, scale, dq, dk, dv, ws, ws_bytes,
                    stream, nullptr, 0);
}

int dsv_sparse_attn_bwd_noalloc(const dsv_problem* p, const void* q, const void* k,
                                const void* v, const void* o, const void* d_o, const float* lse,
                                const int32_t* idx, const int32_t* k_per_head, float scale,
                                float* dq, float* dk, float* dv, void* stream) {
  Geom geo;
  int st = validate_problem(p, k_per_head, &geo);
  if (st != DSV_OK) return st;
  const size_t need = bwd_workspace_bytes(geo);
  // every argument check of the workspace entry point first (no HIP call before them)
  const void* ptrs[] = {q, k, v, o, d_o, lse, idx, dq, dk, dv};
  if ((st = dsv_validate(DSV_OP_BWD, p, k_per_head, DSV_GROUP_SUM, ptrs, 10, need)) != DSV_OK)
    return st;
  if ((st = check_scale(scale)) != DSV_OK) return st;
  if (need > (size_t)DSV_NOALLOC_SCRATCH_BYTES)
    return fail(DSV_ERR_WORKSPACE,
                "backward needs %zu bytes of workspace for its largest head; the no-allocation "
                "entry point has a fixed scratch of %zu bytes",
                need, (size_t)DSV_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (need > 0) {
    const int e = bwd_scratch(&ws);
    if (e) return fail(DSV_ERR_HIP, "scratch lookup failed (hipError %d)", e);
    ws_bytes = (size_t)DSV_NOALLOC_SCRATCH_BYTES;
  }
  return bwd_common(p, q, k, v, o, d_o, lse, idx, k_per_head, scale, dq, dk, dv, ws, ws_bytes,
                    stream, nullptr, 0);
}

int dsv_bwd_chunks(const dsv_problem* p, const int32_t* k_per_head, size_t ws_bytes) {
  Geom geo;
  if (validate_problem(p, k_per_head, &geo) != DSV_OK) return -1;
  if (ws_bytes < bwd_workspace_bytes(geo)) return -1;
  return bwd_chunk_count(geo, ws_bytes);
}

int dsv_sparse_attn_bwd_profiled(const dsv_problem* p, const void* q, const void* k,
                                 const void* v, const void* o, const void* d_o, const float* lse,
                                 const int32_t* idx, const int32_t* k_per_head, float scale,
                                 float* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                                 void* stream, void* const* events, int n_events) {
  if (!events) return fail(DSV_ERR_NULL, "events is NULL");
  return bwd_common(p, q, k, v, o, d_o, lse, idx, k_per_head, scale, dq, dk, dv, ws, ws_bytes,
                    stream, events, n_events);
}

}  // extern "C"
