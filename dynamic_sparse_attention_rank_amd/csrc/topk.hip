// topk.hip — fused low-rank group scoring + exact per-group top-k (critical-KV estimation).
//
// What it computes (DSV summaries, gist.science/{zh,pt,fr,ko}/paper/2502.07590: zh §2.1 low-rank
// estimate of QK^T, zh §2.2 "Fused Kernel" MatMul + Top-K and "Query Grouping"): for every
// (b, h, group g) the k_h keys m with the largest group score
//     sigma[g][m] = (sum_{n in g} Q_lr[n]) . K_lr[m]        (fp32, exact for integer factors)
// with equal scores ranked by the lower key index, written as an ascending row of idx.
// Neither S x S nor NG x S scores are ever stored: scores are recomputed on the fly, in MFMA
// tiles, each time the key stream is traversed.
//
// Design (gfx950):
//   * Workgroup = TK_KW waves over 32 groups of one (b, h). Scores come in 32 x 32 MFMA tiles
//     (v_mfma_f32_32x32x16_bf16) with keys as rows and groups as columns: A is 32 rows of K_lr,
//     loaded straight from memory into registers, and B holds the group sums (each split into
//     two bf16 terms, hi + lo, so that the sums stay exact). Lane l then owns group l % 32 and
//     16 of the 32 keys (rows 8i + 4(l / 32) + j); its partner lane l ^ 32 owns the other 16.
//     Wave kw scores keys 32 kw .. 32 kw + 31 of every TK_TILE-key tile, so the waves split
//     the key stream and share the workgroup's LDS histograms.
//   * Exact selection = radix select on an order-preserving 32-bit image of the fp32 score,
//     8 bits per pass: pass p builds, per group, an LDS histogram of digit p over the keys whose
//     higher digits match the prefix found so far; a wave scan then fixes the digit holding the
//     k-th largest key. A group stops refining as soon as its whole current bin is needed, or
//     when every key counted in the pass had zero bits below the digit (then the bin's keys are
//     all equal). One LDS atomic instruction touches 32 different groups' histograms.
//   * A final pass compacts, per group, the keys above the threshold plus the first `need` keys
//     equal to it, in ascending key order. A lane keeps bit masks of its 16 keys that are above
//     or equal; bit counts of its own and its partner's masks rank a key inside the wave's
//     32-key slice, and per-tile slice counts in LDS give each slice its offset.
//   * Consecutive workgroups go to different XCDs; the block index is remapped so that the
//     workgroups of one (b, h) share an XCD (and its L2) while they stream the same K_lr.
#include <algorithm>

#include "device_common.h"
#include "dsv_internal.h"

namespace dsv {
namespace {

constexpr int TK_GROUPS = 32;              // groups per workgroup (a lane pair each)
constexpr int TK_KW = 16;                  // waves = key slices per workgroup
constexpr int TK_THREADS = 64 * TK_KW;
constexpr int TK_TILE = 32 * TK_KW;        // keys per step of the workgroup
constexpr int TK_HSTRIDE = 257;            // 256 bins + 1 pad word per group histogram
constexpr int TK_SUMW = 4;                 // waves that sum the groups' Q_lr rows

// Order-preserving map float -> uint32 (larger score <=> larger key). -0 is folded onto +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);   // -0 + 0 = +0 (round to nearest)
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Float bounds of a key interval, so that a score is tested against a digit prefix with one
// compare instead of building its key. For finite s: s >= key_lower_bound(k) <=> key(s) >= k,
// and s < key_upper_bound(k) <=> key(s) < k (k up to 2^32; NaN bounds compare false).
__device__ __forceinline__ float key_float(uint32_t key) {   // the float whose key is `key`
  return __uint_as_float(key ^ ((key & 0x80000000u) ? 0x80000000u : 0xffffffffu));
}
__device__ __forceinline__ float key_lower_bound(unsigned long long k) {
  if (k <= 0x007fffffull) return -INFINITY;                 // at or below the key of -inf
  if (k > 0xff800000ull) return __builtin_nanf("");         // above the key of +inf: none
  return key_float((uint32_t)k);
}
__device__ __forceinline__ float key_upper_bound(unsigned long long k) {
  if (k > 0xff800000ull) return INFINITY;                   // every finite score
  if (k <= 0x007fffffull) return -INFINITY;                 // no finite score
  return key_float((uint32_t)k);
}

// The smallest float above a finite x.
__device__ __forceinline__ float next_up(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) == 0u) return __uint_as_float(1u);   // +-0 -> smallest subnormal
  return __uint_as_float((u & 0x80000000u) ? u - 1u : u + 1u);
}

// Contraction layout. bf16: k-step i covers features 16i .. 16i + 15, lane slot h = l / 32 holds
// 16i + 8h .. 16i + 8h + 7 (one 16-byte load). fp32: slot h holds features h R/2 .. h R/2 + R/2 - 1,
// one per v_mfma_f32_32x32x2f32 step (R/8 16-byte loads). A lane's own feature f (< R/2) is
// element f of its loads in both cases.
template <bool F32, int R>
struct TopkCfg {
  static constexpr int ES = F32 ? 4 : 2;             // bytes per element
  static constexpr int RB = R * ES;                  // bytes per row
  static constexpr int NB = F32 ? R / 8 : R / 16;    // 16-byte loads per lane and row
  static constexpr int NF = R / 2;                   // features per lane
  __device__ static int off(int i, int h) { return F32 ? 2 * h * R + 16 * i : 32 * i + 16 * h; }
};

// Block index -> (b, h, group block). Blocks x, x + 8, x + 16, .. run on XCD x % 8; they get
// consecutive logical indices, so that one (b, h)'s blocks share an XCD (and its L2) while they
// stream the same K_lr. Heads go heaviest first.
__device__ __forceinline__ void decode_block(const Geom& geo, int& b, int& h, int& gblock) {
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int logical = xcd * (nblk >> 3) + min(xcd, nblk & 7) + (blockIdx.x >> 3);
  const int gblocks = (geo.NG + TK_GROUPS - 1) / TK_GROUPS;
  const int slot = logical / gblocks;
  gblock = logical - slot * gblocks;
  b = slot / geo.H;
  h = geo.order[slot - b * geo.H];
}

// The score stream of one workgroup: group sums of its 32 groups as B operands, and a walk over
// the key tiles that hands each lane the 16 scores of its group for its keys of every tile.
// Element 4i + j of a lane's scores is key TK_TILE t + 32 kw + 8i + 4 hh + j (lane = 32 hh + g).
template <bool F32, int R>
struct ScoreStream {
  using C = TopkCfg<F32, R>;
  const unsigned char* klr;
  int S, kw, g, hh;
  float ssum[C::NF];
  u32x4 b_hi[F32 ? 1 : C::NB], b_lo[F32 ? 1 : C::NB];

  // Sums the group members' Q_lr rows: waves 0 .. TK_SUMW-1 sum every TK_SUMW-th member of the
  // lane's group into the LDS partials `part`; every wave then adds the partials in the same
  // order (deterministic). Contains two workgroup barriers: every thread calls it.
  __device__ __forceinline__ void init(const Geom& geo, const void* qlr_, const void* klr_, int bh,
                                       int my_group, float* part) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    kw = tid >> 6;
    g = lane & 31;
    hh = lane >> 5;
    S = geo.S;
    const long long head_base = (long long)bh * S * R;   // element offset of (b,h)
    klr = static_cast<const unsigned char*>(klr_) + head_base * C::ES;
    const unsigned char* qlr = static_cast<const unsigned char*>(qlr_) + head_base * C::ES;
    if (kw < TK_SUMW) {
      float ps[C::NF];
#pragma unroll
      for (int f = 0; f < C::NF; ++f) ps[f] = 0.0f;
      if (my_group < geo.NG) {
        const GroupGeom gg{geo.Hh, geo.W, geo.gt, geo.gh, geo.gw, geo.nbh, geo.nbw};
        for (int j = kw; j < geo.G; j += TK_SUMW) {
          const unsigned char* row = qlr + (long long)gg.token(my_group, j) * C::RB;
#pragma unroll
          for (int i = 0; i < C::NB; ++i) {
            const u32x4 v = ld16(row + C::off(i, hh));
            if constexpr (F32) {
#pragma unroll
              for (int e = 0; e < 4; ++e) ps[4 * i + e] += __uint_as_float(v[e]);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                ps[8 * i + 2 * e] += bf16_lo(v[e]);
                ps[8 * i + 2 * e + 1] += bf16_hi(v[e]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int f = 0; f < C::NF; ++f) part[(kw * C::NF + f) * 64 + lane] = ps[f];
    }
    __syncthreads();
#pragma unroll
    for (int f = 0; f < C::NF; ++f) {
      ssum[f] = part[f * 64 + lane];
#pragma unroll
      for (int w = 1; w < TK_SUMW; ++w) ssum[f] += part[(w * C::NF + f) * 64 + lane];
    }
    // bf16 B operands: s = hi + lo with hi = bf16(s), lo = bf16(s - hi); exact while |s| < 2^16
    // for integer sums, and products with bf16 K_lr entries are exact in the fp32 accumulator.
    if constexpr (!F32) {
#pragma unroll
      for (int i = 0; i < C::NB; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float s0 = ssum[8 * i + 2 * e], s1 = ssum[8 * i + 2 * e + 1];
          const float h0 = bf16_round(s0), h1 = bf16_round(s1);
          b_hi[i][e] = pack_bf16(h0, h1);
          b_lo[i][e] = pack_bf16(s0 - h0, s1 - h1);
        }
      }
    }
    __syncthreads();   // partials read: the caller may reuse their LDS
  }

  // A operands: key row TK_TILE t + 32 kw + g of tile t (clamped to the last key; the scores
  // of keys past the end are never used)
  __device__ __forceinline__ void load_a(int t, u32x4* a) const {
    const int m = min(t * TK_TILE + 32 * kw + g, S - 1);
    const unsigned char* krow = klr + (long long)m * C::RB;
#pragma unroll
    for (int i = 0; i < C::NB; ++i) a[i] = ld16(krow + C::off(i, hh));
  }
  // scores of the tile's 32 keys (rows) for the 32 groups (columns), plus c0 (the lane's
  // group's offset: 0, or minus its window base, which keeps integer scores exact)
  float c0 = 0.0f;
  __device__ __forceinline__ floatx16 scores(const u32x4* a) const {
    floatx16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = c0;
#pragma unroll
    for (int i = 0; i < C::NB; ++i) {
      if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma32_f32(__uint_as_float(a[i][e]), ssum[4 * i + e], acc);
      } else {
        acc = mfma32_bf16(a[i], b_hi[i], acc);
        acc = mfma32_bf16(a[i], b_lo[i], acc);
      }
    }
    return acc;
  }
  // Walks the key tiles in order, calling body(scores, t, Flag<partial>): operands are loaded
  // two tiles ahead and scored one tile ahead, so neither the loads nor the MFMAs wait in line.
  template <class Body>
  __device__ __forceinline__ void walk(Body&& body) const {
    const int nfull = S / TK_TILE;   // tiles without keys past the end
    u32x4 a0[C::NB], a1[C::NB];
    load_a(0, a0);
    load_a(1, a1);
    floatx16 acc = scores(a0);
    for (int t = 0; t < nfull; t += 2) {
      load_a(t + 2, a0);
      floatx16 nxt = scores(a1);
      body(acc, t, Flag<false>{});
      acc = nxt;
      if (t + 1 >= nfull) break;
      load_a(t + 3, a1);
      nxt = scores(a0);
      body(acc, t + 1, Flag<false>{});
      acc = nxt;
    }
    if (nfull * TK_TILE < S) body(acc, nfull, Flag<true>{});   // acc holds tile nfull
  }
  // The full tiles j * stride, j < ns (a sample of the key stream), as walk() does.
  template <class Body>
  __device__ __forceinline__ void walk_sample(int ns, int stride, Body&& body) const {
    u32x4 a0[C::NB], a1[C::NB];
    load_a(0, a0);
    load_a(min(1, ns - 1) * stride, a1);
    floatx16 acc = scores(a0);
    for (int j = 0; j < ns; j += 2) {
      load_a(min(j + 2, ns - 1) * stride, a0);
      floatx16 nxt = scores(a1);
      body(acc, j * stride);
      acc = nxt;
      if (j + 1 >= ns) break;
      load_a(min(j + 3, ns - 1) * stride, a1);
      nxt = scores(a0);
      body(acc, (j + 1) * stride);
      acc = nxt;
    }
  }
};

// Threshold window. A sample of the key stream (TK_SAMPLE_TILES tiles spread over it) gives each
// group an estimate of its k-th largest score; one sweep then counts every key into TK_W bins
// of one score unit each around that estimate (plus a bin below and one above the window), so
// for integer-valued scores the bin where the count from the top reaches k holds a single
// score value T, with `need` of its keys still to take. The compaction tests scores against T
// exactly and verifies that it took k keys; a group whose threshold falls outside its window,
// or whose count does not verify (scores that are not integers), is resolved by the radix
// passes instead, which are exact for any scores.
constexpr int TK_W = 512;                  // window bins of one score unit each
constexpr int TK_WSTRIDE = TK_W + 3;       // bins: (below), window, above, pad (3 mod 64)
constexpr int TK_SAMPLE_TILES = 8;         // sampled tiles (8 x 512 keys)
constexpr int TK_SBINS = 256;              // linear bins of the sample histogram

template <bool F32, int R>
__global__ __launch_bounds__(TK_THREADS) void topk_kernel(const void* __restrict__ qlr_,
                                                          const void* __restrict__ klr_,
                                                          int32_t* __restrict__ idx, Geom geo) {
  using C = TopkCfg<F32, R>;
  static_assert(TK_SUMW * 64 * C::NF <= TK_GROUPS * TK_HSTRIDE, "partial sums overflow");
  static_assert(TK_SBINS <= TK_HSTRIDE && TK_W == 8 * 64, "bin layout");
  // group-sum partials first, then the sample histogram, then the radix histograms
  __shared__ uint32_t hist[TK_GROUPS * TK_HSTRIDE];
  __shared__ uint32_t whist[TK_GROUPS * TK_WSTRIDE];   // window counts
  // compaction: per tile parity, group and key slice, the slice's count of keys above the
  // threshold (bits 0..15) and equal to it (bits 16..31)
  __shared__ __attribute__((aligned(16))) uint32_t tcnt[2][TK_GROUPS][TK_KW];
  __shared__ uint32_t st_prefix[TK_GROUPS];
  __shared__ int st_krem[TK_GROUPS];   // keys still to take at the threshold
  // Group state: -1 = no such group; 0..3 = radix refining, that many digits known (and the
  // next histogram pass is that index); 16 + D = radix finished with D digits known;
  // kWindow = threshold value st_t found in the window.
  constexpr int kWindow = 32;
  __shared__ int st_npass[TK_GROUPS];
  __shared__ int st_active[4];
  // per group: set when a key counted in the current radix pass has a nonzero bit below the
  // digit
  __shared__ uint32_t st_lowbits[TK_GROUPS];
  // per group, once the radix passes finish: 1 if the key range left holds a single score
  __shared__ uint32_t st_single[TK_GROUPS];
  __shared__ uint32_t st_mn[TK_GROUPS], st_mx[TK_GROUPS];   // sample extremes (key images)
  __shared__ float st_tlo[TK_GROUPS];   // window base: bin i + 1 counts score st_tlo + i
  __shared__ float st_t[TK_GROUPS];
  __shared__ int st_done[TK_GROUPS];    // row written with exactly k keys
  __shared__ int st_retry;

  const int tid = threadIdx.x;
  const int kw = tid >> 6;       // wave = key slice
  const int lane = tid & 63;
  const int g = lane & 31;       // group of the workgroup
  const int hh = lane >> 5;      // contraction slot / key half

  int b, h, gblock;
  decode_block(geo, b, h, gblock);
  const int bh = b * geo.H + h;
  const int S = geo.S;
  const int kh = geo.k[h];
  const int my_group = gblock * TK_GROUPS + g;

  if (kh == S) {   // dense head: every key, in order, without scoring
    for (int gi = 0; gi < TK_GROUPS && gblock * TK_GROUPS + gi < geo.NG; ++gi) {
      int32_t* row = idx + geo.row_offset(b, h, gblock * TK_GROUPS + gi);
      for (int m = tid; m < S; m += TK_THREADS) row[m] = m;
    }
    return;
  }

  ScoreStream<F32, R> ss;
  ss.init(geo, qlr_, klr_, bh, my_group, reinterpret_cast<float*>(hist));

  for (int i = tid; i < TK_GROUPS; i += TK_THREADS) {
    const bool valid = gblock * TK_GROUPS + i < geo.NG;
    st_prefix[i] = 0;
    st_lowbits[i] = 0;
    st_krem[i] = kh;
    st_npass[i] = valid ? 0 : -1;
    st_done[i] = valid ? 0 : 1;
    st_mn[i] = 0xffffffffu;
    st_mx[i] = 0u;
  }
  for (int i = tid; i < TK_GROUPS * TK_HSTRIDE; i += TK_THREADS) hist[i] = 0;
  for (int i = tid; i < TK_GROUPS * TK_WSTRIDE; i += TK_THREADS) whist[i] = 0;
  __syncthreads();

  // ---- threshold window (a uniform decision: every wave takes the same branches)
  const int nfull = S / TK_TILE;
  const int ns = min(TK_SAMPLE_TILES, nfull);
  if (ns > 0) {
    const int stride = nfull / ns;
    // sample extremes
    float smn = INFINITY, smx = -INFINITY;
    ss.walk_sample(ns, stride, [&](const floatx16& acc, int) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        smn = fminf(smn, acc[e]);
        smx = fmaxf(smx, acc[e]);
      }
    });
    smn = fminf(smn, __shfl_xor(smn, 32, 64));
    smx = fmaxf(smx, __shfl_xor(smx, 32, 64));
    __hip_atomic_fetch_min(&st_mn[g], score_key(smn), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_max(&st_mx[g], score_key(smx), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();
    // sample histogram: TK_SBINS equal bins over [min, max]
    {
      const float mn = key_float(st_mn[g]), mx = key_float(st_mx[g]);
      const float inv = mx > mn ? (float)TK_SBINS / (mx - mn) : 0.0f;
      uint32_t* const hrow = &hist[g * TK_HSTRIDE];
      ss.walk_sample(ns, stride, [&](const floatx16& acc, int) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int bin = min((int)((acc[e] - mn) * inv), TK_SBINS - 1);
          __hip_atomic_fetch_add(&hrow[bin], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      });
    }
    __syncthreads();
    // the estimate: the sample's score at the rank that k takes in the whole row; the window
    // is centred on it
    const int nsamp = ns * TK_TILE;
    const uint32_t rt = (uint32_t)max(1LL, ((long long)nsamp * kh + S - 1) / S);
    for (int gl = kw; gl < TK_GROUPS; gl += TK_KW) {
      if (st_npass[gl] < 0) continue;   // uniform across the wave
      uint32_t* hr = &hist[gl * TK_HSTRIDE];
      uint32_t c[4], lsum = 0;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        c[tt] = hr[TK_SBINS - 1 - (4 * lane + tt)];
        lsum += c[tt];
      }
      uint32_t incl = lsum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t x = __shfl_up(incl, off, 64);
        if (lane >= off) incl += x;
      }
      uint32_t excl = incl - lsum;
      const float mn = key_float(st_mn[gl]), mx = key_float(st_mx[gl]);
      wave_lds_fence();
      if (excl < rt && rt <= incl) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          if (excl + c[tt] >= rt) {
            const int bin = TK_SBINS - 1 - (4 * lane + tt);
            const float est = mx > mn ? mn + ((float)bin + 0.5f) * ((mx - mn) / (float)TK_SBINS)
                                      : mn;
            st_tlo[gl] = floorf(est) - (float)(TK_W / 2);
            break;
          }
          excl += c[tt];
        }
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) hr[4 * lane + tt] = 0;
    }
    __syncthreads();
    // window sweep: scores offset by -tlo in the MFMA accumulator, bins by floor
    ss.c0 = st_npass[g] >= 0 ? -st_tlo[g] : 0.0f;
    uint32_t* const wrow = &whist[g * TK_WSTRIDE];
    ss.walk([&](const floatx16& acc, int t, auto tail_tag) {
      constexpr bool kTail = decltype(tail_tag)::value;
      const int mb = t * TK_TILE + 32 * kw + 4 * hh;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        // keys below the window land in bin 0, which is never read (only the count from the
        // top matters); counting them costs no more than masking them out
        int bin = min(max(__float2int_rd(acc[e]), -1), TK_W) + 1;
        if constexpr (kTail) bin = mb + 8 * (e >> 2) + (e & 3) < S ? bin : 0;
        __hip_atomic_fetch_add(&wrow[bin], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    });
    ss.c0 = 0.0f;
    __syncthreads();
    // the bin where the count from the top reaches k: 8 bins per lane, from the top
    for (int gl = kw; gl < TK_GROUPS; gl += TK_KW) {
      if (st_npass[gl] < 0) continue;   // uniform
      const uint32_t* wr = &whist[gl * TK_WSTRIDE];
      const uint32_t above = wr[TK_W + 1];
      uint32_t c[8], lsum = 0;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        c[tt] = wr[TK_W - (8 * lane + tt)];
        lsum += c[tt];
      }
      uint32_t incl = lsum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t x = __shfl_up(incl, off, 64);
        if (lane >= off) incl += x;
      }
      uint32_t excl = above + incl - lsum;
      incl += above;
      const float tlo = st_tlo[gl];
      const uint32_t k = (uint32_t)kh;
      wave_lds_fence();
      if (above < k && excl < k && k <= incl) {   // otherwise: outside the window (radix)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          if (excl + c[tt] >= k) {
            const int bin = TK_W - (8 * lane + tt);   // counts score tlo + bin - 1
            st_t[gl] = tlo + (float)(bin - 1);
            st_krem[gl] = (int)(k - excl);
            st_npass[gl] = kWindow;
            break;
          }
          excl += c[tt];
        }
      }
    }
    __syncthreads();
  }

  // ---- rounds: radix passes for the groups still refining, then compaction of the rows not
  // yet written; a window row whose count does not verify goes to the radix passes
  for (int round = 0; round < 2; ++round) {
    for (int pass = 0; pass < 4; ++pass) {
      if (tid == 0) {
        int act = 0;
        for (int i = 0; i < TK_GROUPS; ++i) act |= (st_npass[i] == pass);
        st_active[pass] = act;
      }
      __syncthreads();
      if (!st_active[pass]) continue;   // uniform: no group refines in this pass
      // Histogram pass. The lane also ORs the bits below the digit over the keys it counts.
      const int dshift = 24 - 8 * pass;
      const int pshift = 32 - 8 * pass;
      const unsigned long long pfx = st_prefix[g];
      const bool act = st_npass[g] == pass;
      const bool p0 = pass == 0;
      uint32_t* const hrow = &hist[g * TK_HSTRIDE];
      uint32_t lowor = 0;
      // after pass 0: the scores whose keys carry the prefix are those in [lo, hi)
      const float lo = key_lower_bound(pfx << (pshift & 31));
      const float hi = key_upper_bound((pfx + 1) << (pshift & 31));
      auto count = [&](const floatx16& acc, int t, auto tail_tag, auto first_tag) {
        constexpr bool kTail = decltype(tail_tag)::value;
        constexpr bool kFirst = decltype(first_tag)::value;
        const int mb = t * TK_TILE + 32 * kw + 4 * hh;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          bool take = act;
          if constexpr (kTail) take = take && mb + 8 * (e >> 2) + (e & 3) < S;
          if constexpr (!kFirst) take = take && acc[e] >= lo && acc[e] < hi;
          if (take) {
            const uint32_t key = score_key(acc[e]);
            __hip_atomic_fetch_add(&hrow[(key >> dshift) & 255u], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            if constexpr (!kFirst) lowor |= key;
          }
        }
      };
      if (p0) {   // every key of an active group counts; its low bits are not tracked
        ss.walk([&](const floatx16& acc, int t, auto tail) { count(acc, t, tail, Flag<true>{}); });
        lowor = 1u;
      } else {
        ss.walk([&](const floatx16& acc, int t, auto tail) { count(acc, t, tail, Flag<false>{}); });
      }
      if ((lowor & ((1u << dshift) - 1u)) != 0) st_lowbits[g] = 1u;   // any lane: not zero
      __syncthreads();
      // Each wave resolves digit `pass` for some of the groups and clears their histograms.
      for (int gl = kw; gl < TK_GROUPS; gl += TK_KW) {
        if (st_npass[gl] != pass) continue;   // uniform across the wave
        uint32_t* hr = &hist[gl * TK_HSTRIDE];
        uint32_t c[4];
        uint32_t lsum = 0;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          c[tt] = hr[255 - (4 * lane + tt)];
          lsum += c[tt];
        }
        uint32_t incl = lsum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t x = __shfl_up(incl, off, 64);
          if (lane >= off) incl += x;
        }
        const uint32_t krem = (uint32_t)st_krem[gl];
        uint32_t excl = incl - lsum;
        const uint32_t pfx_gl = st_prefix[gl];
        const bool low_gl = st_lowbits[gl] != 0u;
        wave_lds_fence();   // every lane has read the state before one lane rewrites it
        if (excl < krem && krem <= incl) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            if (excl + c[tt] >= krem) {
              const uint32_t bin = 255u - (4u * lane + tt);
              const uint32_t left = krem - excl;   // keys still needed inside `bin`
              st_prefix[gl] = (pass == 0) ? bin : ((pfx_gl << 8) | bin);
              st_krem[gl] = (int)left;
              const bool single = pass == 3 || !low_gl;
              st_npass[gl] = (left == c[tt] || single) ? 16 + pass + 1 : pass + 1;
              st_single[gl] = single ? 1u : 0u;
              break;
            }
            excl += c[tt];
          }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) hr[4 * lane + tt] = 0;
        if (lane == 0) st_lowbits[gl] = 0;
      }
      __syncthreads();
    }

    // ---- compaction of the rows not yet written. Both lanes of a group keep the same
    // running state. Keys above the threshold: score >= f_hi; equal to it: score == f_eq (NaN:
    // none); the first `left` equal keys are taken.
    const int gs = st_npass[g];
    const bool writes = st_done[g] == 0;
    float f_hi, f_eq;
    int left;
    if (gs == kWindow) {
      f_eq = st_t[g];
      f_hi = next_up(f_eq);
      left = st_krem[g];
    } else if (gs >= 16) {
      // radix: the digits fix a key prefix; every key above the prefix's range is taken, and
      // either the whole range is needed (left equals its count) or it holds one score
      const int shift = 32 - 8 * (gs - 16);
      const unsigned long long pfx = st_prefix[g];
      const float lo = key_lower_bound(pfx << shift);
      f_hi = key_lower_bound((pfx + 1) << shift);
      left = st_krem[g];
      const bool single = st_single[g] != 0u;
      f_eq = single ? lo : __builtin_nanf("");
      if (!single) {   // the whole range: above from its lower bound on, nothing equal
        f_hi = lo;
        left = 0;
      }
    } else {   // no such group
      f_hi = INFINITY;
      f_eq = __builtin_nanf("");
      left = 0;
    }
    int cnt = 0;
    int32_t* const orow = idx + geo.row_offset(b, h, gs >= 0 ? my_group : 0);
    ss.walk([&](const floatx16& acc, int t, auto tail_tag) {
      constexpr bool kTail = decltype(tail_tag)::value;
      const int mb = t * TK_TILE + 32 * kw + 4 * hh;
      uint32_t gtm = 0, eqm = 0;   // bit e: element e above / equal
      uint64_t anyeq = 0;          // lanes with an element equal to the threshold
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        bool valid = true;
        if constexpr (kTail) valid = mb + 8 * (e >> 2) + (e & 3) < S;
        gtm |= valid && acc[e] >= f_hi ? 1u << e : 0u;
        anyeq |= __builtin_amdgcn_ballot_w64(valid && acc[e] == f_eq);
      }
      if (anyeq != 0) {   // the same in every lane; most tiles have no key at the threshold
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          bool valid = true;
          if constexpr (kTail) valid = mb + 8 * (e >> 2) + (e & 3) < S;
          eqm |= valid && acc[e] == f_eq ? 1u << e : 0u;
        }
      }
      const uint32_t both = gtm | (eqm << 16);
      const uint32_t pboth = (uint32_t)__shfl_xor((int)both, 32, 64);
      const uint32_t pgtm = pboth & 0xffffu, peqm = pboth >> 16;
      tcnt[t & 1][g][kw] = (uint32_t)(__popc(gtm) + __popc(pgtm)) |
                           ((uint32_t)(__popc(eqm) + __popc(peqm)) << 16);
      __syncthreads();
      uint32_t pre = 0, tot = 0;   // (above, equal) counts of the earlier slices / all slices
#pragma unroll
      for (int w4 = 0; w4 < TK_KW; w4 += 4) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(&tcnt[t & 1][g][w4]);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if (w4 + w < kw) pre += c[w];
          tot += c[w];
        }
      }
      const int pre_gt = (int)(pre & 0xffffu), pre_eq = (int)(pre >> 16);
      const int lft = max(left, 0);
      const int base = cnt + pre_gt + min(lft, pre_eq);
      // the lane's selected keys, one at a time (about 10 % of them)
      const int lr = max(lft - pre_eq, 0);   // equal keys this slice may still take
      if (lr == 0 || (eqm | peqm) == 0u) {
        // No equal key is taken before any of the pair's keys above the threshold: the lane's
        // j-th such key goes to base + j + the partner's keys in the blocks before its own
        // (blocks up to its own for the upper lane). `pw` holds those partner bits shifted so
        // that, for either lane, they are the low (e | 3) + 1 bits.
        const uint32_t pw = hh ? pgtm : (pgtm << 4);
        uint32_t todo = writes ? gtm : 0u;
        int p = base;
        while (todo != 0u) {
          const int e = __builtin_ctz(todo);
          todo &= todo - 1u;
          const int pos = p + __popc(__builtin_amdgcn_ubfe(pw, 0u, (uint32_t)((e | 3) + 1)));
          if (pos < kh) orow[pos] = mb + e + (e & 12);
          ++p;
        }
      } else {
      uint32_t todo = writes ? (gtm | eqm) : 0u;
      while (todo != 0u) {
        const int e = __builtin_ctz(todo);
        todo &= todo - 1u;
        const int i = e >> 2;
        const uint32_t own = (1u << e) - 1u;
        const uint32_t par = (1u << (4 * i + 4 * hh)) - 1u;   // partner blocks before e
        const int gtb = __popc(gtm & own) + __popc(pgtm & par);
        const int eqb = __popc(eqm & own) + __popc(peqm & par);
        const bool sel = ((gtm >> e) & 1u) || eqb < lr;
        const int pos = base + gtb + min(lr, eqb);
        if (sel && pos < kh) orow[pos] = mb + 8 * i + (e & 3);
      }
      }
      cnt += (int)(tot & 0xffffu) + min(lft, (int)(tot >> 16));
      left -= (int)(tot >> 16);
    });
    // verify: a row is done when exactly k keys were taken; otherwise (a window threshold on
    // scores that are not integers) the group is resolved by the radix passes
    if (tid == 0) st_retry = 0;
    __syncthreads();
    if (writes && gs >= 0 && hh == 0 && kw == 0) {
      if (cnt == kh) {
        st_done[g] = 1;
      } else {
        st_npass[g] = 0;
        st_prefix[g] = 0;
        st_krem[g] = kh;
        st_lowbits[g] = 0;
        st_retry = 1;
      }
    }
    __syncthreads();
    if (!st_retry) break;
  }
}

// ---- adaptive k (the "critical KV pairs carry a given share of the attention mass" rule)
//
// A group's k is the smallest number of keys whose softmax weights w_m = exp(ls (sigma_m - M))
// (M = the group's largest score), largest first, reach `mass` of the row's total weight. The
// largest weights belong to the largest scores, so the keys are taken in score order and the
// answer is found by the same radix walk over the order-preserving score image as the top-k:
// every digit bin carries its keys' count and the sum of their weights, each weight evaluated
// in fp64 and rounded to a fixed-point integer u = rint(w 2^P) (P from the host so that a whole
// row sums below 2^63). Integer sums do not depend on the order of the atomics, so the result
// is reproducible bit for bit. Pass 0 (every key) gives the row total Z and the target
// ceil(mass Z); each pass keeps the bin in which the running sum from the top reaches it. When
// that bin holds a single score value T (its keys have no bits below the digit, or all 32 bits
// are fixed), j = ceil((target - sum above T) / u_T) of its keys are needed and k = (keys above
// T) + j.
constexpr int AK_STRIDE = 257;   // 256 bins + 1 pad word per group

template <bool F32, int R>
__global__ __launch_bounds__(TK_THREADS) void adaptive_k_kernel(const void* __restrict__ qlr_,
                                                                const void* __restrict__ klr_,
                                                                AdaptiveParams ap,
                                                                int32_t* __restrict__ k_group,
                                                                int32_t* __restrict__ k_head,
                                                                Geom geo) {
  using C = TopkCfg<F32, R>;
  static_assert(TK_SUMW * 64 * C::NF <= TK_GROUPS * TK_HSTRIDE, "partial sums overflow");
  __shared__ unsigned long long hmass[TK_GROUPS * AK_STRIDE];   // summed fixed-point weights
  __shared__ uint32_t hcnt[TK_GROUPS * TK_HSTRIDE];   // counts; the group sums' partials first
  __shared__ uint32_t st_max[TK_GROUPS];              // order-preserving image of the maximum
  __shared__ uint32_t st_prefix[TK_GROUPS];
  __shared__ int st_npass[TK_GROUPS];                 // as in topk_kernel
  __shared__ uint32_t st_lowbits[TK_GROUPS];
  __shared__ unsigned long long st_above[TK_GROUPS];  // weight of the keys above the prefix
  __shared__ uint32_t st_nabove[TK_GROUPS];           // and their number
  __shared__ unsigned long long st_target[TK_GROUPS];
  __shared__ int st_active[4];

  const int tid = threadIdx.x;
  const int kw = tid >> 6;
  const int lane = tid & 63;
  const int g = lane & 31;
  int b, h, gblock;
  decode_block(geo, b, h, gblock);
  const int my_group = gblock * TK_GROUPS + g;
  const int S = geo.S;

  ScoreStream<F32, R> ss;
  ss.init(geo, qlr_, klr_, b * geo.H + h, my_group, reinterpret_cast<float*>(hcnt));
  for (int i = tid; i < TK_GROUPS * AK_STRIDE; i += TK_THREADS) hmass[i] = 0ull;
  for (int i = tid; i < TK_GROUPS * TK_HSTRIDE; i += TK_THREADS) hcnt[i] = 0u;
  for (int i = tid; i < TK_GROUPS; i += TK_THREADS) {
    st_max[i] = 0u;
    st_prefix[i] = 0u;
    st_lowbits[i] = 0u;
    st_above[i] = 0ull;
    st_nabove[i] = 0u;
    st_target[i] = 0ull;
    st_npass[i] = (gblock * TK_GROUPS + i < geo.NG) ? 0 : -1;
  }
  __syncthreads();

  // ---- the maximum of every group's scores
  float mx = -INFINITY;
  ss.walk([&](const floatx16& acc, int t, auto tail_tag) {
    constexpr bool kTail = decltype(tail_tag)::value;
    const int mb = t * TK_TILE + 32 * ss.kw + 4 * ss.hh;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if constexpr (kTail) {
        if (mb + 8 * (e >> 2) + (e & 3) < S) mx = fmaxf(mx, acc[e]);
      } else {
        mx = fmaxf(mx, acc[e]);
      }
    }
  });
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  __hip_atomic_fetch_max(&st_max[g], score_key(mx), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
  __syncthreads();

  // fixed-point weight of score s in a group with maximum m (fp64, explicit roundings: the
  // bins and the final step must see the very same integer for equal scores)
  auto weight_fx = [&](float s, double m) -> unsigned long long {
    const double w = exp(__dmul_rn(ap.ls, __dsub_rn((double)s, m)));
    return (unsigned long long)rint(__dmul_rn(w, ap.fx));
  };
  const double M64 = (double)key_float(st_max[g]);

  // ---- radix passes with weighted bins
  for (int pass = 0; pass < 4; ++pass) {
    if (tid == 0) {
      int act = 0;
      for (int i = 0; i < TK_GROUPS; ++i) act |= (st_npass[i] == pass);
      st_active[pass] = act;
    }
    __syncthreads();
    if (!st_active[pass]) continue;   // uniform
    const int dshift = 24 - 8 * pass;
    const int pshift = 32 - 8 * pass;
    const unsigned long long pfx = st_prefix[g];
    const bool act = st_npass[g] == pass;
    // after pass 0: the scores whose keys carry the prefix are those in [lo, hi)
    const float lo = key_lower_bound(pfx << (pshift & 31));
    const float hi = key_upper_bound((pfx + 1) << (pshift & 31));
    uint32_t* const crow = &hcnt[g * TK_HSTRIDE];
    unsigned long long* const mrow = &hmass[g * AK_STRIDE];
    uint32_t lowor = 0;
    ss.walk([&](const floatx16& acc, int t, auto tail_tag) {
      constexpr bool kTail = decltype(tail_tag)::value;
      const int mb = t * TK_TILE + 32 * ss.kw + 4 * ss.hh;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        bool take = act;
        if constexpr (kTail) take = take && mb + 8 * (e >> 2) + (e & 3) < S;
        if (pass > 0) take = take && acc[e] >= lo && acc[e] < hi;
        if (take) {
          const uint32_t key = score_key(acc[e]);
          const uint32_t d = (key >> dshift) & 255u;
          __hip_atomic_fetch_add(&crow[d], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          __hip_atomic_fetch_add(&mrow[d], weight_fx(acc[e], M64), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
          lowor |= key;
        }
      }
    });
    // pass 0 does not track the low bits (its bins are never final)
    if (pass == 0 || (lowor & ((1u << dshift) - 1u)) != 0) st_lowbits[g] = 1u;
    __syncthreads();

    // Each wave resolves some of the groups: bins from the top, running sums by a wave scan.
    for (int gl = kw; gl < TK_GROUPS; gl += TK_KW) {
      if (st_npass[gl] != pass) continue;   // uniform across the wave
      unsigned long long m[4], msum = 0ull;
      uint32_t c[4], csum = 0u;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int bin = 255 - (4 * lane + tt);
        m[tt] = hmass[gl * AK_STRIDE + bin];
        c[tt] = hcnt[gl * TK_HSTRIDE + bin];
        msum += m[tt];
        csum += c[tt];
      }
      unsigned long long mincl = msum;
      uint32_t cincl = csum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned long long x = __shfl_up(mincl, off, 64);
        const uint32_t y = __shfl_up(cincl, off, 64);
        if (lane >= off) {
          mincl += x;
          cincl += y;
        }
      }
      unsigned long long target = st_target[gl];
      if (pass == 0) {   // the row total; the target never exceeds it
        const unsigned long long Z = __shfl(mincl, 63, 64);
        const double tz = ceil(__dmul_rn(ap.mass, (double)Z));
        target = tz >= (double)Z ? Z : (unsigned long long)tz;
      }
      const unsigned long long above = st_above[gl];
      const uint32_t nabove = st_nabove[gl];
      const uint32_t pfx_gl = st_prefix[gl];
      const bool lowbits = st_lowbits[gl] != 0u;
      const uint32_t mkey = st_max[gl];
      wave_lds_fence();   // every lane has read the state before one lane rewrites it
      unsigned long long mex = mincl - msum;
      uint32_t cex = cincl - csum;
      if (above + mex < target && target <= above + mincl) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          if (above + mex + m[tt] >= target) {
            const uint32_t bin = 255u - (4u * lane + tt);
            const uint32_t npfx = pass == 0 ? bin : ((pfx_gl << 8) | bin);
            const unsigned long long nabove_m = above + mex;
            const uint32_t nabove_c = nabove + cex;
            if (pass == 3 || !lowbits) {
              // one score value T remains: the keys of the bin are all equal to it
              const uint32_t tkey = npfx << (24 - 8 * pass);
              const unsigned long long uT = weight_fx(key_float(tkey), (double)key_float(mkey));
              const unsigned long long j = (target - nabove_m + uT - 1ull) / uT;
              const int kg = (int)max(1ull, (unsigned long long)nabove_c + j);
              const int grp = gblock * TK_GROUPS + gl;
              if (k_group) k_group[((long long)b * geo.H + h) * geo.NG + grp] = kg;
              atomicMax(&k_head[h], kg);
              st_npass[gl] = 16 + pass + 1;
            } else {
              st_prefix[gl] = npfx;
              st_above[gl] = nabove_m;
              st_nabove[gl] = nabove_c;
              st_npass[gl] = pass + 1;
            }
            break;
          }
          mex += m[tt];
          cex += c[tt];
        }
      }
      if (pass == 0 && lane == 0) st_target[gl] = target;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        hmass[gl * AK_STRIDE + 4 * lane + tt] = 0ull;
        hcnt[gl * TK_HSTRIDE + 4 * lane + tt] = 0u;
      }
      if (lane == 0) st_lowbits[gl] = 0u;
    }
    __syncthreads();
  }
}

// ---- MAX group reduction: sigma[g][m] = max over the members n of g of Q_lr[n] . K_lr[m]
//
// The per-member scores are the literal S x S x r product: one wave owns two groups and keeps
// their members' Q_lr rows as MFMA operands in registers (rows = members, 32 per tile), the
// key rows are the other operand (columns = keys), so a lane holds one key and 16 members:
// the group maximum is an in-lane max and one swap with the partner lane. A wave then runs
// the same exact radix select and ordered compaction as the SUM path on its own two groups
// (lanes 0..31: the first group, 32..63: the second; lane c holds key 32t + c of block t),
// with no workgroup barriers: its histograms and state are its own. Equal bins of one
// instruction are folded by ballots in the first pass, where nearly all keys share a few bins.
// With CACHE, the first pass also stores every group score as its order-preserving key in a
// caller workspace (one row per group; slots s0 .. s0 + gridDim / blocks-per-slot of this
// launch), and the later passes and the compaction read the keys back instead of recomputing
// the 32-member products: one S x S x r product per launch instead of one per pass. A row
// holds segments of 4 key blocks (128 keys): the key of lane c in block t sits at
// 128 (t / 4) + 4c + t % 4, so one 16-byte load gives a lane its keys of 4 blocks. Both
// variants select the same keys.
constexpr int TM_WAVES = 4;
constexpr int TM_THREADS = 64 * TM_WAVES;
constexpr int TM_GROUPS = 2 * TM_WAVES;   // groups per workgroup

template <bool F32, int R, bool CACHE>
__global__ __launch_bounds__(TM_THREADS) void topk_max_kernel(const void* __restrict__ qlr_,
                                                              const void* __restrict__ klr_,
                                                              int32_t* __restrict__ idx,
                                                              Geom geo, int s0,
                                                              uint32_t* __restrict__ cache) {
  using C = TopkCfg<F32, R>;
  __shared__ uint32_t hist[TM_GROUPS * TK_HSTRIDE];
  __shared__ uint32_t st_prefix[TM_GROUPS];
  __shared__ int st_krem[TM_GROUPS];
  __shared__ int st_npass[TM_GROUPS];   // as in topk_kernel
  __shared__ uint32_t st_lowbits[TM_GROUPS];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int c32 = lane & 31;
  const int hh = lane >> 5;
  // block -> (b, h, group block), one (b, h)'s blocks on one XCD, heavy heads first
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int logical = xcd * (nblk >> 3) + min(xcd, nblk & 7) + (blockIdx.x >> 3);
  const int gblocks = (geo.NG + TM_GROUPS - 1) / TM_GROUPS;
  const int lslot = logical / gblocks;   // slot inside this launch
  const int gblock = logical - lslot * gblocks;
  const int slot = s0 + lslot;
  const int b = slot / geo.H;
  const int h = geo.order[slot - b * geo.H];
  const int S = geo.S;
  const int kh = geo.k[h];
  const int g0 = gblock * TM_GROUPS + 2 * w;   // the wave's groups g0, g0 + 1
  if (g0 >= geo.NG) return;                    // the whole wave; there are no barriers
  const int gl = 2 * w + hh;                   // the lane's group, local index
  const int my_g = g0 + hh;
  const bool gvalid = my_g < geo.NG;
  const long long head_base = ((long long)b * geo.H + h) * S * R;
  const unsigned char* klr = static_cast<const unsigned char*>(klr_) + head_base * C::ES;
  const unsigned char* qlr = static_cast<const unsigned char*>(qlr_) + head_base * C::ES;

  if (kh == S) {   // dense head: every key, in order, without scoring
    for (int gi = 0; gi < 2 && g0 + gi < geo.NG; ++gi) {
      int32_t* row = idx + geo.row_offset(b, h, g0 + gi);
      for (int m = lane; m < S; m += 64) row[m] = m;
    }
    return;
  }

  // ---- member operands: tile qt of group g0 + gw holds members 32 qt + c32 (rows); members
  // past G are zero rows whose scores are masked below
  const int G = geo.G;
  const int nqt = (G + 31) >> 5;
  u32x4 qa[2][2][C::NB];
  const GroupGeom gg{geo.Hh, geo.W, geo.gt, geo.gh, geo.gw, geo.nbh, geo.nbw};
#pragma unroll
  for (int gw = 0; gw < 2; ++gw)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int j = 32 * qt + c32;
      const bool ok = g0 + gw < geo.NG && j < G;
      const unsigned char* row = qlr + (long long)(ok ? gg.token(g0 + gw, j) : 0) * C::RB;
#pragma unroll
      for (int i = 0; i < C::NB; ++i)
        qa[gw][qt][i] = ok ? ld16(row + C::off(i, hh)) : u32x4{0u, 0u, 0u, 0u};
    }

  // ---- key operands of block t (key 32t + c32, clamped) and the block's group maxima:
  // lane c of half hh gets sigma[g0 + hh][32t + c]
  auto load_k = [&](int t, u32x4* kb) {
    const int m = min(32 * t + c32, S - 1);
    const unsigned char* krow = klr + (long long)m * C::RB;
#pragma unroll
    for (int i = 0; i < C::NB; ++i) kb[i] = ld16(krow + C::off(i, hh));
  };
  auto block_max = [&](const u32x4* kb) -> float {
    float mx[2];
#pragma unroll
    for (int gw = 0; gw < 2; ++gw) {
      mx[gw] = -INFINITY;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        if (qt >= nqt) break;   // uniform: G <= 32 has one member tile
        floatx16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int i = 0; i < C::NB; ++i) {
          if constexpr (F32) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc = mfma32_f32(__uint_as_float(qa[gw][qt][i][e]), __uint_as_float(kb[i][e]), acc);
          } else {
            acc = mfma32_bf16(qa[gw][qt][i], kb[i], acc);
          }
        }
        if (32 * qt + 32 > G) {   // uniform: rows (members) 32 qt + 8i + 4hh + j past G
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * qt + 8 * (e >> 2) + 4 * hh + (e & 3) >= G) acc[e] = -INFINITY;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) mx[gw] = fmaxf(mx[gw], acc[e]);
      }
    }
    const float m0 = fmaxf(mx[0], __shfl_xor(mx[0], 32, 64));
    const float m1 = fmaxf(mx[1], __shfl_xor(mx[1], 32, 64));
    return hh ? m1 : m0;
  };
  const int nblocks = (S + 31) >> 5;
  // the lane's row of cached keys (its group's; a lane of an absent second group reads the
  // first group's row and its results are discarded); rows of nseg segments of 128 keys
  const int nseg = (nblocks + 3) >> 2;
  uint32_t* const crow =
      CACHE ? cache + ((long long)lslot * geo.NG + (gvalid ? my_g : g0)) * (128LL * nseg)
            : nullptr;
  // body(score, t): loads two blocks ahead, scores one block ahead
  auto walk = [&](auto&& body) {
    u32x4 k0[C::NB], k1[C::NB];
    load_k(0, k0);
    load_k(1, k1);
    float sc = block_max(k0);
    for (int t = 0; t < nblocks; t += 2) {
      load_k(t + 2, k0);
      float nx = block_max(k1);
      body(sc, t);
      sc = nx;
      if (t + 1 >= nblocks) break;
      load_k(t + 3, k1);
      nx = block_max(k0);
      body(sc, t + 1);
      sc = nx;
    }
  };

  // the later walks: cached keys, U segments (4U blocks) of loads in flight; a lane reads back
  // only the positions it stored itself (blocks past the last one: never used)
  auto walk_cached = [&](auto&& body) {
    constexpr int U = 4;
    for (int T0 = 0; T0 < nseg; T0 += U) {
      u32x4 u[U];
#pragma unroll
      for (int i = 0; i < U; ++i)
        u[i] = ld16(crow + 128LL * min(T0 + i, nseg - 1) + 4 * c32);
#pragma unroll
      for (int i = 0; i < U; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * (T0 + i) + e;
          if (t < nblocks) body(key_float(u[i][e]), t);   // uniform
        }
    }
  };
  auto walk_later = [&](auto&& body) {
    if constexpr (CACHE)
      walk_cached(body);
    else
      walk(body);
  };

  if (c32 == 0) {
    st_prefix[gl] = 0;
    st_lowbits[gl] = 0;
    st_krem[gl] = kh;
    st_npass[gl] = gvalid ? 0 : -1;
  }
  for (int i = lane; i < 2 * TK_HSTRIDE; i += 64) hist[2 * w * TK_HSTRIDE + i] = 0;
  wave_lds_fence();
  uint32_t* const hrow = &hist[gl * TK_HSTRIDE];

  for (int pass = 0; pass < 4; ++pass) {
    const bool act = st_npass[gl] == pass;
    if (__ballot(act) == 0) continue;   // uniform: neither group refines in this pass
    const int dshift = 24 - 8 * pass;
    const int pshift = 32 - 8 * pass;
    const unsigned long long pfx = st_prefix[gl];
    const float lo = key_lower_bound(pfx << (pshift & 31));
    const float hi = key_upper_bound((pfx + 1) << (pshift & 31));
    uint32_t lowor = 0;
    if (pass == 0) {
      // nearly every key falls into a few bins: one atomic per distinct (group, bin)
      walk([&](const float sc, const int t) {
        if constexpr (CACHE)
          if (gvalid) crow[128 * (t >> 2) + 4 * c32 + (t & 3)] = score_key(sc);
        const bool take = act && 32 * t + c32 < S;
        const uint32_t bin = score_key(sc) >> 24;
        unsigned long long todo = __ballot(take);
        while (todo) {
          const int l0 = __builtin_ctzll(todo);
          const uint32_t b0 = __builtin_amdgcn_readlane(bin, l0);
          const unsigned long long m = __ballot(take && bin == b0 && hh == (l0 >> 5));
          if (lane == l0)
            __hip_atomic_fetch_add(&hist[(2 * w + (l0 >> 5)) * TK_HSTRIDE + b0],
                                   (uint32_t)__popcll(m), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
          todo &= ~m;
        }
      });
      lowor = 1u;   // not tracked in the first pass
      if constexpr (CACHE) __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    } else {
      walk_later([&](const float sc, const int t) {
        if (act && 32 * t + c32 < S && sc >= lo && sc < hi) {
          const uint32_t key = score_key(sc);
          __hip_atomic_fetch_add(&hrow[(key >> dshift) & 255u], 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
          lowor |= key;
        }
      });
    }
    uint32_t o = lowor & ((1u << dshift) - 1u);
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) o |= __shfl_xor(o, off, 64);
    if (c32 == 0 && o != 0) st_lowbits[gl] = 1u;
    wave_lds_fence();
    // resolve digit `pass` of each of the wave's groups that refined in it
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int glr = 2 * w + gi;
      if (st_npass[glr] != pass) continue;   // uniform
      uint32_t* hr = &hist[glr * TK_HSTRIDE];
      uint32_t c[4];
      uint32_t lsum = 0;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        c[tt] = hr[255 - (4 * lane + tt)];
        lsum += c[tt];
      }
      uint32_t incl = lsum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t x = __shfl_up(incl, off, 64);
        if (lane >= off) incl += x;
      }
      const uint32_t krem = (uint32_t)st_krem[glr];
      uint32_t excl = incl - lsum;
      wave_lds_fence();   // every lane has read the state before one lane rewrites it
      if (excl < krem && krem <= incl) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          if (excl + c[tt] >= krem) {
            const uint32_t bin = 255u - (4u * lane + tt);
            const uint32_t left = krem - excl;
            st_prefix[glr] = (pass == 0) ? bin : ((st_prefix[glr] << 8) | bin);
            st_krem[glr] = (int)left;
            st_npass[glr] = (left == c[tt] || pass == 3 || st_lowbits[glr] == 0)
                                ? 16 + pass + 1 : pass + 1;
            break;
          }
          excl += c[tt];
        }
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) hr[4 * lane + tt] = 0;
      wave_lds_fence();
      if (lane == 0) st_lowbits[glr] = 0;
      wave_lds_fence();
    }
  }

  // ---- compaction: keys above the threshold plus the first `left` equal to it, in key order
  const int gs = st_npass[gl];
  const unsigned long long pfx = gs >= 16 ? st_prefix[gl] : 0xffffffffull;
  const int shift = gs >= 16 ? 32 - 8 * (gs - 16) : 0;
  const float f_hi = key_lower_bound((pfx + 1) << shift);
  const float f_hi_u = key_upper_bound((pfx + 1) << shift);
  const float f_lo = key_lower_bound(pfx << shift);
  int left = gs >= 16 ? st_krem[gl] : 0;
  int cnt = 0;
  int32_t* const orow = idx + geo.row_offset(b, h, gvalid ? my_g : g0);
  const uint32_t below = (1u << c32) - 1u;
  walk_later([&](const float sc, const int t) {
    const int m = 32 * t + c32;
    const bool valid = m < S;
    const bool gt = valid && sc >= f_hi;
    const bool eq = valid && sc >= f_lo && sc < f_hi_u;
    const uint32_t gth = (uint32_t)(__ballot(gt) >> (32 * hh));
    const uint32_t eqh = (uint32_t)(__ballot(eq) >> (32 * hh));
    const int lft = max(left, 0);
    const int eqb = __popc(eqh & below);
    const bool sel = gt || (eq && eqb < lft);
    const int pos = cnt + __popc(gth & below) + min(lft, eqb);
    if (sel && gvalid && pos < kh) orow[pos] = m;
    cnt += __popc(gth) + min(lft, __popc(eqh));
    left -= __popc(eqh);
  });
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

size_t topk_max_cache_slot_bytes(const Geom& geo) {
  const size_t row = ((size_t)geo.S + 127) / 128 * 128;   // whole 128-key segments
  return ((size_t)geo.NG * row * sizeof(uint32_t) + 255) & ~(size_t)255;
}

int launch_topk(const Geom& geo, const void* q_lr, const void* k_lr, int reduce, int32_t* idx,
                void* ws, size_t ws_bytes, void* stream) {
  const bool mx = reduce == DSV_GROUP_MAX;
  const int gpb = mx ? TM_GROUPS : TK_GROUPS;
  const int gblocks = (geo.NG + gpb - 1) / gpb;
  const int nslots = geo.B * geo.H;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool f32 = geo.dtype == DSV_FP32;
  // MAX with a workspace for at least one slot's scores: chunks of slots that fit it
  const size_t per_slot = topk_max_cache_slot_bytes(geo);
  const int cslots = (mx && ws && reinterpret_cast<uintptr_t>(ws) % 256 == 0)
                         ? (int)std::min<size_t>((size_t)nslots, ws_bytes / per_slot)
                         : 0;
  uint32_t* cache = static_cast<uint32_t*>(ws);
#define DSV_TOPK_CASE(F, RR)                                                                    \
  if (f32 == F && geo.r == RR) {                                                                \
    if (mx && cslots > 0) {                                                                     \
      for (int s0 = 0; s0 < nslots; s0 += cslots) {                                             \
        const int n = std::min(cslots, nslots - s0);                                            \
        hipLaunchKernelGGL((topk_max_kernel<F, RR, true>), dim3(n * gblocks),                   \
                           dim3(TM_THREADS), 0, st, q_lr, k_lr, idx, geo, s0, cache);           \
      }                                                                                         \
    } else if (mx) {                                                                            \
      hipLaunchKernelGGL((topk_max_kernel<F, RR, false>), dim3(nslots * gblocks),               \
                         dim3(TM_THREADS), 0, st, q_lr, k_lr, idx, geo, 0, nullptr);            \
    } else {                                                                                    \
      hipLaunchKernelGGL((topk_kernel<F, RR>), dim3(nslots * gblocks), dim3(TK_THREADS), 0, st, \
                         q_lr, k_lr, idx, geo);                                                 \
    }                                                                                           \
    return (int)hipGetLastError();                                                              \
  }
  DSV_TOPK_CASE(false, 16)
  DSV_TOPK_CASE(false, 32)
  DSV_TOPK_CASE(false, 48)
  DSV_TOPK_CASE(false, 64)
  DSV_TOPK_CASE(true, 16)
  DSV_TOPK_CASE(true, 32)
  DSV_TOPK_CASE(true, 48)
  DSV_TOPK_CASE(true, 64)
#undef DSV_TOPK_CASE
  return (int)hipErrorInvalidValue;
}

}  // namespace dsv

namespace dsv {

int launch_adaptive_k(const Geom& geo, const void* q_lr, const void* k_lr,
                      const AdaptiveParams& ap, int32_t* k_group, int32_t* k_head, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(fill_i32_kernel, dim3((geo.H + 255) / 256), dim3(256), 0, st, k_head, geo.H,
                     0);
  const int gblocks = (geo.NG + TK_GROUPS - 1) / TK_GROUPS;
  const dim3 grid(geo.B * geo.H * gblocks);
  const bool f32 = geo.dtype == DSV_FP32;
#define DSV_AK_CASE(F, RR)                                                                     \
  if (f32 == F && geo.r == RR) {                                                               \
    hipLaunchKernelGGL((adaptive_k_kernel<F, RR>), grid, dim3(TK_THREADS), 0, st, q_lr, k_lr, \
                       ap, k_group, k_head, geo);                                              \
    return (int)hipGetLastError();                                                             \
  }
  DSV_AK_CASE(false, 16)
  DSV_AK_CASE(false, 32)
  DSV_AK_CASE(false, 48)
  DSV_AK_CASE(false, 64)
  DSV_AK_CASE(true, 16)
  DSV_AK_CASE(true, 32)
  DSV_AK_CASE(true, 48)
  DSV_AK_CASE(true, 64)
#undef DSV_AK_CASE
  return (int)hipErrorInvalidValue;
}

}  // namespace dsv
