// dsv_internal.h — host-side geometry shared by the C ABI layer and the kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/dsv.h"

#if defined(__HIP__) || defined(__HIPCC__)
#define DSV_HD __host__ __device__
#else
#define DSV_HD
#endif

namespace dsv {

constexpr int kMaxHeads = 128;

// Everything a kernel needs to locate its work, passed by value as a kernel argument.
struct Geom {
  int B, H, T, Hh, W, S, d, r, gt, gh, gw, G, NG, nbh, nbw;
  int dtype;
  long long ksum;            // sum_h k_h
  int k[kMaxHeads];          // k_h
  long long pre[kMaxHeads];  // sum_{h'<h} k_h'
  int order[kMaxHeads];      // launch order: the planner's order for one device (cost ~ k_h)

  // Start of row (b, h, g) in the packed idx array.
  DSV_HD inline long long row_offset(int b, int h, int g) const {
    return (long long)NG * ((long long)b * ksum + pre[h]) + (long long)g * k[h];
  }
};

// The planner's processing order (dsv_plan.cpp): heads by decreasing cost, equal costs by
// lower head index. With one device it is also the order in which the kernels launch heads.
void lpt_order(const double* cost, int n, int* order);

// Validation (HIP-free). Fills `geo` when the problem is valid.
int validate_problem(const dsv_problem* p, const int32_t* k_per_head, Geom* geo);
void set_error(const char* fmt, ...);

// Adaptive k: per-key softmax weights exp(ls * (sigma - max)) in fp64, rounded to integer
// multiples of 1 / fx (fx = 2^P, P = 62 - bit length of S, so a whole row sums below 2^63).
struct AdaptiveParams {
  double ls;     // logit scale (the caller's fp32 value)
  double fx;     // 2^P
  double mass;   // share of the row's weight the group's k keys must carry, in (0, 1]
};
// Fixed-point exponent P of the adaptive-k weights for a row of S keys.
inline int adaptive_fx_bits(int S) {
  int bl = 0;
  while (bl < 31 && (1u << bl) <= (unsigned)S) ++bl;   // bit length of S
  return 62 - bl;
}

// Kernel launchers (one per translation unit). Return 0 or a hipError_t value.
// reduce = MAX uses ws (when 256-byte aligned and at least one slot's worth) to keep the group
// scores between passes, processing as many (b, h) slots per launch as fit.
int launch_topk(const Geom& geo, const void* q_lr, const void* k_lr, int reduce, int32_t* idx,
                void* ws, size_t ws_bytes, void* stream);
size_t topk_max_cache_slot_bytes(const Geom& geo);   // NG rows of S keys (4 bytes each) in
                                                     // 128-key segments, 256-aligned
int launch_adaptive_k(const Geom& geo, const void* q_lr, const void* k_lr,
                      const AdaptiveParams& ap, int32_t* k_group, int32_t* k_head, void* stream);
int launch_attn_fwd(const Geom& geo, const void* q, const void* k, const void* v,
                    const int32_t* idx, float scale, void* o, float* lse, void* stream);
// `events` (may be NULL): 4 hipEvent_t per head chunk, recorded around the chunk's stages.
int launch_attn_bwd(const Geom& geo, const void* q, const void* k, const void* v, const void* o,
                    const void* d_o, const float* lse, const int32_t* idx, float scale, float* dq,
                    float* dk, float* dv, void* ws, size_t ws_bytes, void* stream,
                    void* const* events);
// Minimum device workspace of the backward (bf16 path): the bucket tables and staging rows
// of the heaviest (b, h) slot (per (group, selected key) edge: an int16 dV row and dK row,
// two fp32 steps and a bucket-list entry). Larger workspaces let a launch cover more slots.
size_t bwd_workspace_bytes(const Geom& geo);
// Number of head chunks (launch groups) the backward uses with this workspace (1 on fp32).
int bwd_chunk_count(const Geom& geo, size_t ws_bytes);
// Device address of the no-allocation backward's scratch array (DSV_NOALLOC_SCRATCH_BYTES) on
// the calling thread's current device, looked up on the first call per device. 0 or a
// hipError_t value.
int bwd_scratch(void** ptr);

}  // namespace dsv
