// attn_fwd.hip — query-grouped sparse attention, forward.
//
// For query n of group g (DSV summaries, gist.science/{zh,pt,fr,ko}/paper/2502.07590: zh §2.1
// "sparse computation" — full attention on the critical KV pairs only; zh §2.2 "Query
// Grouping" — the group's queries share one index list):
//     O[n] = sum_{m in idx(g)} softmax_m(scale * q_n . k_m) v_m,   LSE[n] = log sum_m exp(...)
//
// bf16 path (gfx950 MFMA): one wave per group (G = 16..64 queries, d = 64 or 128).
//   * The group's Q is held in registers as the B operand of S^T = K Q^T
//     (v_mfma_f32_16x16x32_bf16), so each 16x16 score tile gives a lane one query and 4 keys.
//   * Keys are consumed in chunks of 32 from the ascending index row. A lane gathers K rows in
//     16-byte pieces straight into MFMA operand registers; V rows are gathered one full
//     256-byte row per 16 lanes and transposed in registers (v_perm_b32) into the A operand of
//     O^T += V^T P^T. The key order inside the contraction is permuted so that the P^T operand
//     is exactly the score tile a lane already holds: no LDS and no cross-lane traffic on the
//     hot loop except the occasional max reduction.
//   * Online softmax in the log2 domain with an fp32 running max and sum; the max is only
//     raised (and O rescaled) when a new score exceeds it by more than 2^8, which keeps exp2
//     arguments <= 8 and makes rescaling rare. Results are exact regardless of when it is raised.
//   * The next chunk's K/V rows are requested while the current chunk is still being
//     computed (indices one chunk further ahead).
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

template <int D>
struct VRaw;   // one lane's slice of 8 V rows: DPL = D/16 consecutive features per row
template <>
struct VRaw<128> {
  u32x4 r[8];
};
template <>
struct VRaw<64> {
  u32x2 r[8];
};

template <int D>
struct FwdChunk {
  u32x4 k[2][D / 32];   // K rows (16kb + li), features 32ks + 8lg .. +8
  VRaw<D> v;            // V rows of this lane's 8 keys, features DPL*li .. +DPL
};

struct ChunkKeys {
  int kk[2];   // key index for K rows 16kb + li
  int vk[8];   // key index for this lane's 8 V rows
};

template <int D, int QB>
__global__ __launch_bounds__(64) void attn_fwd_bf16(const uint16_t* __restrict__ q,
                                                    const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v,
                                                    const int32_t* __restrict__ idx, float scale,
                                                    uint16_t* __restrict__ o,
                                                    float* __restrict__ lse, Geom geo) {
  constexpr int DPL = D / 16;   // features per lane per V row; also O^T dimension blocks
  constexpr int KS = D / 32;    // contraction steps of S^T = K Q^T
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

  int tok[QB];
  u32x4 qop[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    tok[qb] = gg.token(g, qb * 16 + li);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[qb][ks] = ld16(Q + (long long)tok[qb] * D + ks * 32 + 8 * lg);
  }

  floatx4 oacc[QB][DPL];
  float mrun[QB], lrun[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrun[qb] = -INFINITY;
    lrun[qb] = 0.f;
#pragma unroll
    for (int f = 0; f < DPL; ++f) oacc[qb][f] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = scale * kLog2e;

  auto load_keys = [&](int cb, ChunkKeys& ck) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) ck.kk[kb] = clamp_key(row[min(cb + 16 * kb + li, kh - 1)], geo.S);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = cb + (e < 4 ? 4 * lg + e : 16 + 4 * lg + (e - 4));
      ck.vk[e] = clamp_key(row[min(p, kh - 1)], geo.S);
    }
  };
  auto load_k = [&](const ChunkKeys& ck, FwdChunk<D>& ch) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ch.k[kb][ks] = ld16(K + (long long)ck.kk[kb] * D + ks * 32 + 8 * lg);
  };
  auto load_v = [&](const ChunkKeys& ck, FwdChunk<D>& ch) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (D == 128)
        ch.v.r[e] = ld16(V + (long long)ck.vk[e] * D + DPL * li);
      else
        ch.v.r[e] = ld8(V + (long long)ck.vk[e] * D + DPL * li);
    }
  };

  // One K/V buffer: the next chunk's K rows are requested as soon as the score MFMAs have
  // consumed the current ones, and its V rows right after the current V has been
  // transposed, so both loads overlap the softmax and the P.V MFMAs. Indices run one chunk
  // further ahead.
  ChunkKeys keys_nx;
  FwdChunk<D> ch;
  {
    ChunkKeys k0;
    load_keys(0, k0);
    load_k(k0, ch);
    load_v(k0, ch);
    load_keys(32, keys_nx);   // clamped reads stay inside the row even when k <= 32
  }
  for (int cb = 0; cb < kh; cb += 32) {
    const bool more = cb + 32 < kh;
    floatx4 s[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a = mfma_bf16(ch.k[kb][ks], qop[qb][ks], a);
        s[kb][qb] = a;
      }
    if (more) load_k(keys_nx, ch);
    // V^T operand: vA[f] = feature DPL*li + f of the lane's 8 keys
    u32x4 vA[DPL];
    if constexpr (D == 128)
      transpose8x8_b16(ch.v.r, vA);
    else
      transpose8x4_b16(ch.v.r, vA);
    if (more) {
      load_v(keys_nx, ch);
      load_keys(cb + 64, keys_nx);
    }
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
        for (int f = 0; f < DPL; ++f) oacc[qb][f] *= alpha;
      }
      float p[2][4];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[kb][j] = exp2f(t[kb][j] - mrun[qb]);
          psum += p[kb][j];
        }
      lrun[qb] += psum;
      // P^T operand: element e <-> key (e < 4 ? 4lg + e : 16 + 4lg + e - 4), matching vA
      u32x4 pb;
      pb[0] = pack_bf16(p[0][0], p[0][1]);
      pb[1] = pack_bf16(p[0][2], p[0][3]);
      pb[2] = pack_bf16(p[1][0], p[1][1]);
      pb[3] = pack_bf16(p[1][2], p[1][3]);
#pragma unroll
      for (int f = 0; f < DPL; ++f) oacc[qb][f] = mfma_bf16(vA[f], pb, oacc[qb][f]);
    }
  }

  // finalise: full row sums, normalise, store O (bf16) and LSE (fp32)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l = wave_xor_sum(lrun[qb], 16);
    l = wave_xor_sum(l, 32);
    const float inv = 1.0f / l;
    uint16_t* orow = o + base + (long long)tok[qb] * D;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // dims DPL*(4lg + j) + f, f = 0..DPL-1
      if constexpr (D == 128) {
        u32x4 w;
#pragma unroll
        for (int f2 = 0; f2 < 4; ++f2)
          w[f2] = pack_bf16(oacc[qb][2 * f2][j] * inv, oacc[qb][2 * f2 + 1][j] * inv);
        *reinterpret_cast<u32x4*>(orow + DPL * (4 * lg + j)) = w;
      } else {
        u32x2 w;
#pragma unroll
        for (int f2 = 0; f2 < 2; ++f2)
          w[f2] = pack_bf16(oacc[qb][2 * f2][j] * inv, oacc[qb][2 * f2 + 1][j] * inv);
        *reinterpret_cast<u32x2*>(orow + DPL * (4 * lg + j)) = w;
      }
    }
    if (lg == 0)
      lse[((long long)b * geo.H + h) * geo.S + tok[qb]] = (mrun[qb] + log2f(l)) * kLn2;
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
