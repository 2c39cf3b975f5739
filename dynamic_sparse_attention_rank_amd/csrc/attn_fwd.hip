// attn_fwd.hip — query-grouped sparse attention, forward.
//
// For query n of group g (DSV summaries, gist.science/{zh,pt,fr,ko}/paper/2502.07590: zh §2.1
// "sparse computation" — full attention on the critical KV pairs only; zh §2.2 "Query
// Grouping" — the group's queries share one index list):
//     O[n] = sum_{m in idx(g)} softmax_m(scale * q_n . k_m) v_m,   LSE[n] = log sum_m exp(...)
//
// bf16 path (gfx950 MFMA): one wave per group (G = 16..64 queries, d = 64 or 128).
//   * The group's Q rows sit in LDS (one swizzled copy); S^T = K Q^T reads them as 16-byte B
//     operands, so a 16x16 score tile gives a lane one query and 4 keys.
//   * Keys are consumed in chunks of 32 from the ascending index row. K and V rows are both
//     gathered in 16-byte pieces straight into MFMA operand registers (lane: one key, 8
//     features). The V^T operand of O^T += V^T P^T is made from those registers by an MFMA
//     against a 0/1 selection matrix (exact), with the key order chosen so that the P^T
//     operand is exactly the score tile a lane already holds.
//   * Online softmax in the log2 domain with an fp32 running max and sum; the max is only
//     raised (and O rescaled) when a new score exceeds it by more than 2^8, which keeps exp2
//     arguments <= 8 and makes rescaling rare. Results are exact regardless of when it is raised.
//   * The next chunk's K/V rows are requested as soon as the current ones have been turned
//     into operands, and the key indices one chunk further ahead; every load in the loop is
//     unconditional (positions clamped), so the waits for them are exact.
// fp32 path: plain fp32 FMA per lane (one lane per query); it exists for fp32 inputs and is
// not tuned.
#include <math.h>

#include "device_common.h"
#include "dsv_internal.h"

namespace dsv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRaise = 8.0f;   // log2-domain slack before the running max is raised

__device__ __forceinline__ void decode_unit(const Geom& geo, int unit, int& b, int& h, int& g) {
  const int per_head = geo.B * geo.NG;
  const int slot = unit / per_head;
  const int rem = unit - slot * per_head;
  h = geo.order[slot];
  b = rem / geo.NG;
  g = rem - b * geo.NG;
}

template <int D, int QB>
__global__ __launch_bounds__(64) void attn_fwd_bf16(const uint16_t* __restrict__ q,
                                                    const uint16_t* k,   // k, v: not restrict,
                                                    const uint16_t* v,   // see the prefetch
                                                    const int32_t* __restrict__ idx, float scale,
                                                    uint16_t* __restrict__ o,
                                                    float* __restrict__ lse, Geom geo) {
  constexpr int NDB = D / 16;   // feature blocks of O^T
  constexpr int KS = D / 32;    // contraction steps of S^T = K Q^T
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint16_t qn[16 * QB * D];
  const int lane = threadIdx.x;
  const int lg = lane >> 4;
  const int li = lane & 15;
  int b, h, g;
  decode_unit(geo, blockIdx.x, b, h, g);
  const int kh = geo.k[h];
  const long long base = ((long long)b * geo.H + h) * geo.S * D;
  const uint16_t* Q = q + base;
  const uint16_t* K = k + base;
  const uint16_t* V = v + base;
  const int32_t* row = idx + geo.row_offset(b, h, g);
  const GroupGeom gg{geo.Hh, geo.W, geo.gt, geo.gh, geo.gw, geo.nbh, geo.nbw};

  // ---- the group's Q rows into LDS (CPR lanes per row, one 16-byte chunk each)
  {
    const int rr = lane / CPR, c = lane % CPR;
    for (int r0 = 0; r0 < 16 * QB; r0 += 64 / CPR) {
      const int r = r0 + rr;
      const int n = gg.token(g, r);
      *reinterpret_cast<u32x4*>(&qn[swz<D>(r, 8 * c)]) = ld16(Q + (long long)n * D + 8 * c);
    }
  }
  __syncthreads();

  floatx4 oacc[QB][NDB];
  float mrun[QB], lrun[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrun[qb] = -INFINITY;
    lrun[qb] = 0.f;
#pragma unroll
    for (int f = 0; f < NDB; ++f) oacc[qb][f] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = scale * kLog2e;
  u32x4 sel[2];
  make_selection(lane, sel);

  u32x4 kb_n[2][KS], vb_n[2][KS];   // K / V rows 16kb + li of the current chunk, features
  int nkey[2];                      // 32ks + 8lg ..; keys of the chunk after the next one
  auto load_keys = [&](int cb, int out[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) out[kb] = row[min(cb + 16 * kb + li, kh - 1)];
  };
  auto load_nat = [&](const int keys[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = clamp_key(keys[kb], geo.S);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kb_n[kb][ks] = ld16(K + (long long)key * D + ks * 32 + 8 * lg);
        vb_n[kb][ks] = ld16(V + (long long)key * D + ks * 32 + 8 * lg);
      }
    }
  };
  {
    int k0[2];
    load_keys(0, k0);
    load_nat(k0);
    load_keys(32, nkey);
  }

  for (int cb = 0; cb < kh; cb += 32) {
    // ---- S^T = K Q^T ; lane: query 16qb + li, keys 16kb + 4lg + j
    floatx4 s[2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      s[0][qb] = s[1][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 qop = *reinterpret_cast<const u32x4*>(&qn[swz<D>(16 * qb + li, 32 * ks + 8 * lg)]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb][qb] = mfma_bf16(kb_n[kb][ks], qop, s[kb][qb]);
      }
    }
    // ---- V^T operands: row li <-> feature 16fb + li, slot (lg, e) <-> key 4lg + e (e < 4),
    // 16 + 4lg + e - 4 (e >= 4), from the V rows in registers (selection MFMA, exact)
    u32x4 vT[NDB];
#pragma unroll
    for (int fb = 0; fb < NDB; ++fb) {
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      const floatx4 t0 = mfma_bf16(vb_n[0][fb >> 1], sel[fb & 1], z);
      const floatx4 t1 = mfma_bf16(vb_n[1][fb >> 1], sel[fb & 1], z);
      vT[fb] = u32x4{pack_bf16(t0[0], t0[1]), pack_bf16(t0[2], t0[3]), pack_bf16(t1[0], t1[1]),
                     pack_bf16(t1[2], t1[3])};
    }
    // K/V registers consumed: request the next chunk (past the end the clamped positions
    // reload the last key; those loads are never used) and the keys of the one after. The
    // compiler barrier keeps the loads after the MFMAs above, so the two K/V buffers are
    // never live together.
    asm volatile("" ::: "memory");
    load_nat(nkey);
    load_keys(cb + 64, nkey);

    const bool tail = cb + 32 > kh;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float t[2][4];
      float lmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x = s[kb][qb][j] * c2;
          if (tail && cb + 16 * kb + 4 * lg + j >= kh) x = -INFINITY;
          t[kb][j] = x;
          lmax = fmaxf(lmax, x);
        }
      if (__ballot(lmax > mrun[qb] + kRaise)) {
        float cmax = wave_xor_max(lmax, 16);
        cmax = wave_xor_max(cmax, 32);
        const float mnew = fmaxf(mrun[qb], cmax);
        const float alpha = exp2f(mrun[qb] - mnew);
        mrun[qb] = mnew;
        lrun[qb] *= alpha;
#pragma unroll
        for (int f = 0; f < NDB; ++f) oacc[qb][f] *= alpha;
      }
      float p[2][4];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[kb][j] = __builtin_amdgcn_exp2f(t[kb][j] - mrun[qb]);
          psum += p[kb][j];
        }
      lrun[qb] += psum;
      // P^T operand: element e <-> key (e < 4 ? 4lg + e : 16 + 4lg + e - 4), matching vT
      const u32x4 pb = {pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                        pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};
#pragma unroll
      for (int fb = 0; fb < NDB; ++fb) oacc[qb][fb] = mfma_bf16(vT[fb], pb, oacc[qb][fb]);
    }
  }

  // finalise: full row sums, normalise, store O (bf16) and LSE (fp32). Lane: query
  // 16qb + li, features 16fb + 4lg + j.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l = wave_xor_sum(lrun[qb], 16);
    l = wave_xor_sum(l, 32);
    const float inv = 1.0f / l;
    const int n = gg.token(g, 16 * qb + li);
    uint16_t* orow = o + base + (long long)n * D;
#pragma unroll
    for (int fb = 0; fb < NDB; ++fb)
      *reinterpret_cast<u32x2*>(orow + 16 * fb + 4 * lg) =
          u32x2{pack_bf16(oacc[qb][fb][0] * inv, oacc[qb][fb][1] * inv),
                pack_bf16(oacc[qb][fb][2] * inv, oacc[qb][fb][3] * inv)};
    if (lg == 0)
      lse[((long long)b * geo.H + h) * geo.S + n] = (mrun[qb] + log2f(l)) * kLn2;
  }
}

// fp32 inputs: one lane per query, exact online softmax, fp32 FMA.
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32(const float* __restrict__ q,
                                                   const float* __restrict__ k,
                                                   const float* __restrict__ v,
                                                   const int32_t* __restrict__ idx, float scale,
                                                   float* __restrict__ o, float* __restrict__ lse,
                                                   Geom geo) {
  const int lane = threadIdx.x;
  int b, h, g;
  decode_unit(geo, blockIdx.x, b, h, g);
  if (lane >= geo.G) return;
  const int kh = geo.k[h];
  const long long base = ((long long)b * geo.H + h) * geo.S * D;
  const int32_t* row = idx + geo.row_offset(b, h, g);
  const GroupGeom gg{geo.Hh, geo.W, geo.gt, geo.gh, geo.gw, geo.nbh, geo.nbw};
  const int n = gg.token(g, lane);
  float qv[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = q[base + (long long)n * D + c] * scale;
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int p = 0; p < kh; ++p) {
    const long long kr = base + (long long)clamp_key(row[p], geo.S) * D;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) s = fmaf(qv[c], k[kr + c], s);
    const float mn = fmaxf(m, s);
    const float alpha = expf(m - mn);
    const float e = expf(s - mn);
    l = l * alpha + e;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] = fmaf(e, v[kr + c], acc[c] * alpha);
    m = mn;
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int c = 0; c < D; ++c) o[base + (long long)n * D + c] = acc[c] * inv;
  lse[((long long)b * geo.H + h) * geo.S + n] = m + logf(l);
}

}  // namespace

int launch_attn_fwd(const Geom& geo, const void* q, const void* k, const void* v,
                    const int32_t* idx, float scale, void* o, float* lse, void* stream) {
  const dim3 grid(geo.B * geo.H * geo.NG);
  const dim3 block(64);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (geo.dtype == DSV_FP32) {
#define DSV_FWD32(DD)                                                                        \
  if (geo.d == DD) {                                                                         \
    hipLaunchKernelGGL((attn_fwd_f32<DD>), grid, block, 0, st, (const float*)q,              \
                       (const float*)k, (const float*)v, idx, scale, (float*)o, lse, geo);   \
    return (int)hipGetLastError();                                                           \
  }
    DSV_FWD32(64)
    DSV_FWD32(128)
#undef DSV_FWD32
    return (int)hipErrorInvalidValue;
  }
  const int QBn = geo.G / 16;
#define DSV_FWD16(DD, QQ)                                                                       \
  if (geo.d == DD && QBn == QQ) {                                                               \
    hipLaunchKernelGGL((attn_fwd_bf16<DD, QQ>), grid, block, 0, st, (const uint16_t*)q,         \
                       (const uint16_t*)k, (const uint16_t*)v, idx, scale, (uint16_t*)o, lse,   \
                       geo);                                                                    \
    return (int)hipGetLastError();                                                              \
  }
  DSV_FWD16(64, 1) DSV_FWD16(64, 2) DSV_FWD16(64, 3) DSV_FWD16(64, 4)
  DSV_FWD16(128, 1) DSV_FWD16(128, 2) DSV_FWD16(128, 3) DSV_FWD16(128, 4)
#undef DSV_FWD16
  return (int)hipErrorInvalidValue;
}

}  // namespace dsv
