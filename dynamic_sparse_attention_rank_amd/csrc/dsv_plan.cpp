// dsv_plan.cpp — host-side planning: head placement over devices (longest-processing-time
// greedy with the sparse imbalance ratio) and the per-head dense-versus-sparse choice.
// No HIP calls: these run on the CPU before anything is enqueued.
#include <math.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "dsv_internal.h"

namespace dsv {

// Longest-processing-time order: heads by decreasing cost, equal costs by lower head index.
void lpt_order(const double* cost, int n, int* order) {
  std::iota(order, order + n, 0);
  std::stable_sort(order, order + n, [&](int a, int b) { return cost[a] > cost[b]; });
}

}  // namespace dsv

using namespace dsv;

extern "C" {

int dsv_plan_order(const int32_t* k_per_head, int32_t heads, double fixed_cost,
                   double cost_per_k, int32_t* order) {
  if (!k_per_head || !order) {
    set_error("k_per_head and order must not be NULL");
    return DSV_ERR_NULL;
  }
  if (heads <= 0) {
    set_error("heads = %d must be positive", heads);
    return DSV_ERR_SHAPE;
  }
  if (!(fixed_cost >= 0.0) || !(cost_per_k >= 0.0) || !isfinite(fixed_cost) ||
      !isfinite(cost_per_k)) {
    set_error("costs must be finite and non-negative");
    return DSV_ERR_SHAPE;
  }
  std::vector<double> cost(heads);
  for (int h = 0; h < heads; ++h) cost[h] = fixed_cost + cost_per_k * (double)k_per_head[h];
  std::vector<int> o(heads);
  lpt_order(cost.data(), heads, o.data());
  for (int i = 0; i < heads; ++i) order[i] = o[i];
  return DSV_OK;
}

int dsv_plan_heads(const int32_t* k_per_head, int32_t heads, int32_t n_parts, double fixed_cost,
                   double cost_per_k, int32_t* part_of_head, double* part_load, double* rho) {
  if (!k_per_head || !part_of_head) {
    set_error("k_per_head and part_of_head must not be NULL");
    return DSV_ERR_NULL;
  }
  if (heads <= 0 || n_parts <= 0) {
    set_error("heads = %d and n_parts = %d must be positive", heads, n_parts);
    return DSV_ERR_SHAPE;
  }
  if (!(fixed_cost >= 0.0) || !(cost_per_k >= 0.0) || !(fixed_cost + cost_per_k > 0.0) ||
      !isfinite(fixed_cost) || !isfinite(cost_per_k)) {
    set_error("costs must be finite, non-negative and not both zero");
    return DSV_ERR_SHAPE;
  }
  for (int h = 0; h < heads; ++h)
    if (k_per_head[h] < 1) {
      set_error("k_per_head[%d] = %d must be >= 1", h, k_per_head[h]);
      return DSV_ERR_K;
    }
  std::vector<double> cost(heads);
  for (int h = 0; h < heads; ++h) cost[h] = fixed_cost + cost_per_k * (double)k_per_head[h];
  std::vector<int> order(heads);
  lpt_order(cost.data(), heads, order.data());
  std::vector<double> load(n_parts, 0.0);
  for (int h : order) {
    int best = 0;
    for (int q = 1; q < n_parts; ++q)
      if (load[q] < load[best]) best = q;
    part_of_head[h] = best;
    load[best] += cost[h];
  }
  double total = 0.0, mx = 0.0;
  for (int q = 0; q < n_parts; ++q) {
    total += load[q];
    mx = std::max(mx, load[q]);
  }
  if (part_load)
    for (int q = 0; q < n_parts; ++q) part_load[q] = load[q];
  if (rho) *rho = mx / (total / (double)n_parts);
  return DSV_OK;
}

// Measured on one MI355X at S = 64K (B=1, H=24, d=128, r=32, G=64, k = 10 % of S):
// top-k 1.30 ms over 24 * 1024 * 65536 scores; forward 6.30 ms and backward 31.3 ms over
// 1.611e8 edges (one step, every slot of the backward in one launch, all of its kernels).
// The estimator's work per score scales with r (two bf16 MFMA terms per 16 features and a
// fixed per-score selection cost, taken here as proportional), the attention's per edge
// with G * d.
int dsv_default_cost_model(const dsv_problem* p, int with_backward, dsv_cost_model* cm) {
  if (!cm) {
    set_error("cm is NULL");
    return DSV_ERR_NULL;
  }
  Geom geo;
  const int32_t one = 1;
  std::vector<int32_t> k1(p ? std::max(p->heads, 1) : 1, one);
  const int st = validate_problem(p, k1.data(), &geo);
  if (st != DSV_OK) return st;
  const double topk_ns = 1.30e6 / (24.0 * 1024.0 * 65536.0);
  const double fwd_ns = 6.30e6 / 1.611e8, bwd_ns = 31.3e6 / 1.611e8;
  cm->topk_ns_per_score = topk_ns * (double)geo.r / 32.0;
  cm->attn_ns_per_edge =
      (with_backward ? fwd_ns + bwd_ns : fwd_ns) * (double)geo.G * geo.d / (64.0 * 128.0);
  return DSV_OK;
}

int dsv_dispatch_k(const dsv_problem* p, const int32_t* k_in, const dsv_cost_model* cm,
                   int32_t* k_out, int32_t* n_dense) {
  if (!cm || !k_out) {
    set_error("cm and k_out must not be NULL");
    return DSV_ERR_NULL;
  }
  Geom geo;
  const int st = validate_problem(p, k_in, &geo);
  if (st != DSV_OK) return st;
  if (!(cm->topk_ns_per_score >= 0.0) || !(cm->attn_ns_per_edge > 0.0) ||
      !isfinite(cm->topk_ns_per_score) || !isfinite(cm->attn_ns_per_edge)) {
    set_error("cost model: topk_ns_per_score >= 0 and attn_ns_per_edge > 0, both finite");
    return DSV_ERR_SHAPE;
  }
  int nd = 0;
  const double S = (double)geo.S;
  for (int h = 0; h < geo.H; ++h) {
    const double sparse = S * cm->topk_ns_per_score + (double)k_in[h] * cm->attn_ns_per_edge;
    const double dense = S * cm->attn_ns_per_edge;
    const bool d = dense <= sparse;
    k_out[h] = d ? geo.S : k_in[h];
    nd += d;
  }
  if (n_dense) *n_dense = nd;
  return DSV_OK;
}

}  // extern "C"
