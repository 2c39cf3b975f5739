// attn_fwd.hip — query-grouped sparse attention, forward.
//
// For query n of group g (DSV summaries, gist.science/{zh,pt,fr,ko}/paper/2502.07590: zh §2.1
// "sparse computation" — full attention on the critical KV pairs only; zh §2.2 "Query
// Grouping" — the group's queries share one index list):
//     O[n] = sum_{m in idx(g)} softmax_m(scale * q_n . k_m) v_m,   LSE[n] = log sum_m exp(...)
//
// bf16 path (gfx950 MFMA): one wave per group (G = 16..64 queries, d = 64 or 128).
//   * The group's Q rows are staged once in LDS (one swizzled copy) and read from there into
//     registers as the B operands of S^T = K Q^T for the whole index row; a 16x16 score tile
//     gives a lane one query and 4 keys.
//   * Keys are consumed in chunks of 32 from the ascending index row. The chunk's K and V rows
//     are gathered into an LDS tile by direct-to-LDS loads that cover whole rows (full cache
//     lines, about twice the gather rate of operand-shaped 64-byte pieces); K operands are
//     swizzled row reads, the V^T operand of O^T += V^T P^T comes from transposed LDS reads of
//     the same rows, so P^T and V^T share the tile's row order.
//   * Online softmax in the log2 domain with an fp32 running max and sum; the max is only
//     raised (and O rescaled) when a new score exceeds it by more than 2^8, which keeps exp2
//     arguments <= 8 and makes rescaling rare. Results are exact regardless of when it is raised.
//   * The next chunk's rows are requested as soon as the current ones are in registers; every
//     lane loads the indices of its own row loads one chunk further ahead. Every load in the
//     loop is unconditional (positions clamped), so no conditional memory operation makes the
//     compiler wait early. The tile is read after all of the wave's loads have retired.
//   * Built with MFMA results in VGPRs: the rare rescale multiplies the O accumulators with
//     VALU ops, and AGPR accumulators would be copied to VGPRs on every chunk.
// fp32 path: v_mfma_f32_16x16x4_f32 tiles, one wave per group, keys in chunks of 16 through
// LDS; it exists for fp32 inputs and is not tuned for speed.
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
  __shared__ __attribute__((aligned(16))) uint16_t kvs[2][32 * D];   // K, V rows of a chunk
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

  // ---- K and V rows of a 32-key chunk go to LDS by direct-to-LDS loads that each cover
  // whole rows (full cache lines: 16-byte pieces, GPR per row, RPI rows per load), about twice
  // the gather rate of loads shaped like MFMA operands (16 rows x 64 bytes). Load i, lane l
  // fills LDS row p = RPI i + l / GPR, stored piece l % GPR (the XOR swizzle swz, so that
  // operand reads do not conflict). Row p holds the chunk's key NI (p % RPI) + p / RPI, which
  // makes a lane's NI keys adjacent in the index row. The score tile's rows are LDS rows, and
  // the V^T operands are transposed reads of the same rows, so P^T and V^T agree on the key
  // order without knowing it; only the tail mask maps a row back to its key.
  constexpr int GPR = D / 8;     // 16-byte pieces per row
  constexpr int RPI = 64 / GPR;  // rows per load
  constexpr int NI = 32 / RPI;   // loads per array and chunk
  const int la = lane / GPR;
  const int lp = lane % GPR;
  // key indices: the NI keys of a lane's row loads (chunk positions NI la + i, adjacent in the
  // index row; positions past the row end read its last key) are loaded a chunk ahead
  struct Keys { uint32_t k[NI]; };
  auto load_keys = [&](int cb) {
    Keys r;
#pragma unroll
    for (int i = 0; i < NI; ++i) r.k[i] = (uint32_t)row[min(cb + NI * la + i, kh - 1)];
    return r;
  };
  Keys kq;   // keys of the next chunk to fetch
  const char* Kb = reinterpret_cast<const char*>(K);
  const char* Vb = reinterpret_cast<const char*>(V);
  auto fetch_rows = [&](const Keys& kr) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int p = RPI * i + la;
      // clamped here, a chunk after the key loads were issued, so that they are not waited for
      // (as unsigned values, see clamp_key: with a signed clamp, same loads in the same order,
      // this loop missed L2 on 60% more of the rows and took 6.39 against 6.28 ms at S = 64K)
      const uint32_t off = (uint32_t)clamp_key((int)kr.k[i], geo.S) * (uint32_t)(2 * D) +
                           (uint32_t)((lp ^ (p % GPR)) << 4);
      global_load_lds16(Kb + off, &kvs[0][RPI * i * D]);
      global_load_lds16(Vb + off, &kvs[1][RPI * i * D]);
    }
  };
  fetch_rows(load_keys(0));
  kq = load_keys(32);
  // the Q operands (B of S^T = K Q^T: query 16qb + li, features 32ks + 8lg ..) stay in
  // registers for the whole row instead of being re-read from LDS every chunk
  u32x4 qop[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[qb][ks] = *reinterpret_cast<const u32x4*>(&qn[swz<D>(16 * qb + li, 32 * ks + 8 * lg)]);

  // mrun is the running maximum of the raw scores q.k (c2 > 0 turns them into log2 units):
  // P = exp2(c2 s - c2 mrun) is then one FMA and one exp2 per score
  const float raise_s = kRaise / c2;
  auto chunk = [&](const int cb, auto tail_tag) {
    constexpr bool kTail = decltype(tail_tag)::value;
    // this chunk's rows are in LDS once all of the wave's loads have retired (the key loads
    // issued after them are then in too)
    wait_vmcnt<0>();
    // ---- operands: K rows 16kb + li (A of S^T = K Q^T, features 32ks + 8lg ..) and V^T
    // (row li <-> feature 16fb + li, slot (lg, e) <-> LDS row 4lg + e (e < 4) or
    // 16 + 4lg + e - 4 (e >= 4)) by transposed reads
    u32x4 ka[2][KS], vT[NDB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[kb][ks] = *reinterpret_cast<const u32x4*>(&kvs[0][swz<D>(16 * kb + li, 32 * ks + 8 * lg)]);
#pragma unroll
    for (int fb = 0; fb < NDB; ++fb) {
      const int r = 4 * lg + (li >> 2), c = 16 * fb + 4 * (li & 3);
      const u32x2 lo = lds_read_tr16(&kvs[1][swz<D>(r, c)]);
      const u32x2 hi = lds_read_tr16(&kvs[1][swz<D>(r + 16, c)]);
      vT[fb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    // operands are in registers: refill the buffer with the next chunk (past the end the
    // clamped positions reload the last key; never used) and fetch the keys after it
    wave_lds_fence();
    fetch_rows(kq);
    kq = load_keys(cb + 64);

    // ---- S^T = K Q^T ; lane: query 16qb + li, LDS rows (keys) 16kb + 4lg + j
    floatx4 s[2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      s[0][qb] = s[1][qb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb][qb] = mfma_bf16(ka[kb][ks], qop[qb][ks], s[kb][qb]);
    }

    // each lane's maximum raw score per query tile; in the last, partial chunk the rows past
    // the end of the index row (LDS row p holds chunk key NI (p % RPI) + p / RPI) are -inf
    float lmax[QB];
    bool raise = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      lmax[qb] = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (kTail) {
            const int p = 16 * kb + 4 * lg + j;
            if (cb + NI * (p % RPI) + p / RPI >= kh) s[kb][qb][j] = -INFINITY;
          }
          lmax[qb] = fmaxf(lmax[qb], s[kb][qb][j]);
        }
      raise = raise || lmax[qb] > mrun[qb] + raise_s;
    }
    // Lazy rescaling: a query's running maximum moves only when a score exceeds it by more
    // than kRaise (so exp2 of the shifted scores stays below 2^kRaise). One uniform branch
    // per chunk keeps the exponentials and the P V^T products below in one basic block.
    if (__ballot(raise)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (__ballot(lmax[qb] > mrun[qb] + raise_s)) {
          float cmax = wave_xor_max(lmax[qb], 16);
          cmax = wave_xor_max(cmax, 32);
          const float mnew = fmaxf(mrun[qb], cmax);
          const float alpha = exp2f((mrun[qb] - mnew) * c2);
          mrun[qb] = mnew;
          lrun[qb] *= alpha;
#pragma unroll
          for (int f = 0; f < NDB; ++f) oacc[qb][f] *= alpha;
        }
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float nm = -mrun[qb] * c2;
      float p[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) p[kb][j] = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][j], c2, nm));
      // pairwise: seven adds in a tree of depth three
      lrun[qb] += ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) +
                  ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
      // P^T operand: element e <-> key (e < 4 ? 4lg + e : 16 + 4lg + e - 4), matching vT
      const u32x4 pb = {pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                        pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};
#pragma unroll
      for (int fb = 0; fb < NDB; ++fb) oacc[qb][fb] = mfma_bf16(vT[fb], pb, oacc[qb][fb]);
    }
  };
  int cb = 0;
  for (; cb + 32 <= kh; cb += 32) chunk(cb, Flag<false>{});
  if (cb < kh) chunk(cb, Flag<true>{});
  // the last chunk requested rows past the end into the other buffer: they land before
  // the workgroup ends and its LDS is handed to another
  wait_vmcnt<0>();

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
      lse[((long long)b * geo.H + h) * geo.S + n] = (mrun[qb] * c2 + log2f(l)) * kLn2;
  }
}

// fp32 inputs: v_mfma_f32_16x16x4_f32 tiles, one wave per group, keys in chunks of 16. The
// group's Q rows and each chunk's K and V rows sit in LDS (rows padded by one word so that the
// operand reads of 16 rows spread over the banks). S^T = K Q^T gives a lane 4 keys of one
// query; the online softmax runs per chunk in the natural-log domain with the scale applied
// to the scores; P^T goes through an LDS tile [key][query] to become the B operand of
// O^T += V^T P^T. Exact up to fp32 rounding; kept simple (it serves fp32 inputs).
template <int D, int QB>
__global__ __launch_bounds__(64) void attn_fwd_f32(const float* __restrict__ q,
                                                   const float* __restrict__ k,
                                                   const float* __restrict__ v,
                                                   const int32_t* __restrict__ idx, float scale,
                                                   float* __restrict__ o, float* __restrict__ lse,
                                                   Geom geo) {
  constexpr int G = 16 * QB;
  constexpr int DP = D + 1;   // LDS row stride of Q, K, V (words)
  constexpr int GP = G + 1;   // LDS row stride of the P tile
  constexpr int NDB = D / 16;
  __shared__ float sq[G * DP];
  __shared__ float sk[16 * DP];
  __shared__ float sv[16 * DP];
  __shared__ float sp[16 * GP];
  const int lane = threadIdx.x;
  const int lg = lane >> 4;
  const int li = lane & 15;
  int b, h, g;
  decode_unit(geo, blockIdx.x, b, h, g);
  const int kh = geo.k[h];
  const long long base = ((long long)b * geo.H + h) * geo.S * D;
  const int32_t* row = idx + geo.row_offset(b, h, g);
  const GroupGeom gg{geo.Hh, geo.W, geo.gt, geo.gh, geo.gw, geo.nbh, geo.nbw};
  for (int i = lane; i < G * D; i += 64) {
    const int r = i / D, c = i - r * D;
    sq[r * DP + c] = q[base + (long long)gg.token(g, r) * D + c];
  }
  floatx4 oacc[QB][NDB];
  float mrun[QB], lrun[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mrun[qb] = -INFINITY;
    lrun[qb] = 0.f;
#pragma unroll
    for (int f = 0; f < NDB; ++f) oacc[qb][f] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  for (int cb = 0; cb < kh; cb += 16) {
    // lane li's key (positions past the row end read its last key; their scores are masked)
    const int key = clamp_key(row[min(cb + li, kh - 1)], geo.S);
    for (int r = 0; r < 16; ++r) {
      const long long kr = base + (long long)__shfl(key, r, 64) * D;
      for (int c = lane; c < D; c += 64) {
        sk[r * DP + c] = k[kr + c];
        sv[r * DP + c] = v[kr + c];
      }
    }
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // S^T: lane holds keys 4lg + j of the chunk for query 16qb + li
      floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int st = 0; st < D / 4; ++st)
        s = mfma_f32(sk[li * DP + 4 * st + lg], sq[(16 * qb + li) * DP + 4 * st + lg], s);
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[j] = cb + 4 * lg + j < kh ? s[j] * scale : -INFINITY;
        tmax = fmaxf(tmax, s[j]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mnew = fmaxf(mrun[qb], tmax);   // finite: key cb is always in the row
      const float alpha = expf(mrun[qb] - mnew);   // 0 on the first chunk
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = expf(s[j] - mnew);
        psum += p;
        sp[(4 * lg + j) * GP + 16 * qb + li] = p;
      }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      lrun[qb] = fmaf(lrun[qb], alpha, psum);
      mrun[qb] = mnew;
#pragma unroll
      for (int f = 0; f < NDB; ++f) oacc[qb][f] *= alpha;
    }
    // O^T += V^T P^T (the P tile is this wave's own LDS writes, read back in order)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int f = 0; f < NDB; ++f)
#pragma unroll
        for (int st = 0; st < 4; ++st)
          oacc[qb][f] = mfma_f32(sv[(4 * st + lg) * DP + 16 * f + li],
                                 sp[(4 * st + lg) * GP + 16 * qb + li], oacc[qb][f]);
    __syncthreads();   // the next chunk's rows overwrite the tiles
  }
  // lane: query 16qb + li, features 16f + 4lg + j
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float inv = 1.0f / lrun[qb];
    const long long n = gg.token(g, 16 * qb + li);
#pragma unroll
    for (int f = 0; f < NDB; ++f)
      *reinterpret_cast<floatx4*>(o + base + n * D + 16 * f + 4 * lg) = oacc[qb][f] * inv;
    if (lg == 0) lse[((long long)b * geo.H + h) * geo.S + n] = mrun[qb] + logf(lrun[qb]);
  }
}

}  // namespace

int launch_attn_fwd(const Geom& geo, const void* q, const void* k, const void* v,
                    const int32_t* idx, float scale, void* o, float* lse, void* stream) {
  const dim3 grid(geo.B * geo.H * geo.NG);
  const dim3 block(64);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (geo.dtype == DSV_FP32) {
    const int QB32 = geo.G / 16;
#define DSV_FWD32(DD, QQ)                                                                    \
  if (geo.d == DD && QB32 == QQ) {                                                           \
    hipLaunchKernelGGL((attn_fwd_f32<DD, QQ>), grid, block, 0, st, (const float*)q,          \
                       (const float*)k, (const float*)v, idx, scale, (float*)o, lse, geo);   \
    return (int)hipGetLastError();                                                           \
  }
    DSV_FWD32(64, 1) DSV_FWD32(64, 2) DSV_FWD32(64, 3) DSV_FWD32(64, 4)
    DSV_FWD32(128, 1) DSV_FWD32(128, 2) DSV_FWD32(128, 3) DSV_FWD32(128, 4)
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
