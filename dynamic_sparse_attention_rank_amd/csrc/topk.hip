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
//   * Workgroup = TK_GW x TK_KW waves over 16 TK_GW groups of one (b, h). Wave (gw, kw) scores
//     groups 16 gw .. 16 gw + 15 against keys 16 kw .. 16 kw + 15 of every TK_TILE-key tile, so
//     the TK_KW waves of a group block split the key stream and share its LDS histograms. The
//     16-row A operand of v_mfma_f32_16x16x32_bf16 holds the group sums (split into two bf16
//     terms, hi + lo, so that the sums stay exact); the B operand (16 keys of K_lr) is loaded
//     straight from memory into registers, one tile ahead. Each 16x16 output tile gives a lane
//     one key and four groups.
//   * Exact selection = radix select on an order-preserving 32-bit image of the fp32 score,
//     8 bits per pass: pass p builds, per group, an LDS histogram of digit p over the keys whose
//     higher digits match the prefix found so far; a wave scan then fixes the digit holding the
//     k-th largest key. A group stops refining as soon as its whole current bin is needed.
//     Lane li adds its four groups' counts in the rotated order (j + li) mod 4, so one LDS
//     atomic instruction touches 16 different groups (at most 4 lanes per histogram) even when
//     all scores fall into the same bin, as they do for the exponent byte of pass 0.
//   * A final pass compacts, per group, the keys above the threshold plus the first `need` keys
//     equal to it, in ascending key order: wave ballots rank a lane's key inside its 16-key
//     slice, and per-tile slice counts in LDS give each slice its offset.
//   * Consecutive workgroups go to different XCDs; the block index is remapped so that the
//     workgroups of one (b, h) share an XCD (and its L2) while they stream the same K_lr.
#include "device_common.h"
#include "dsv_internal.h"

namespace dsv {
namespace {

constexpr int TK_GW = 2;                   // group waves per workgroup (16 groups each)
constexpr int TK_KW = 4;                   // key slices per workgroup (16 keys of a tile each)
constexpr int TK_WAVES = TK_GW * TK_KW;
constexpr int TK_THREADS = 64 * TK_WAVES;
constexpr int TK_GROUPS = 16 * TK_GW;      // groups per workgroup
constexpr int TK_TILE = 16 * TK_KW;        // keys per step of the workgroup
constexpr int TK_HSTRIDE = 257;            // 256 bins + 1 pad word per group histogram

// Order-preserving map float -> uint32 (larger score <=> larger key). -0 is folded onto +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);   // -0 + 0 = +0 (round to nearest)
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

template <bool F32, int R>
struct TopkCfg {
  static constexpr int ES = F32 ? 4 : 2;             // bytes per element
  static constexpr int RB = R * ES;                  // bytes per K_lr row
  static constexpr int KSTEPS = F32 ? R / 4 : (R + 31) / 32;   // MFMA contraction steps
};

template <bool F32, int R>
__global__ __launch_bounds__(TK_THREADS) __attribute__((amdgpu_waves_per_eu(6))) void topk_kernel(const void* __restrict__ qlr_,
                                                          const void* __restrict__ klr_,
                                                          int32_t* __restrict__ idx, Geom geo) {
  using C = TopkCfg<F32, R>;
  __shared__ uint32_t hist[TK_GROUPS * TK_HSTRIDE];
  // compaction: per tile parity, group and key slice, the slice's count of keys above the
  // threshold (bits 0..15) and equal to it (bits 16..31)
  __shared__ __attribute__((aligned(16))) uint32_t tcnt[2][TK_GROUPS][TK_KW];
  __shared__ uint32_t st_prefix[TK_GROUPS];
  __shared__ int st_krem[TK_GROUPS];
  // Group state: -1 = no such group; 0..3 = still refining, that many digits known (and the
  // next histogram pass is that index); 16 + D = finished with D digits known.
  __shared__ int st_npass[TK_GROUPS];
  __shared__ int st_active[4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lg = lane >> 4;
  const int li = lane & 15;
  const int gw = wave / TK_KW;
  const int kw = wave - gw * TK_KW;

  // block -> (b, h, group block): blocks x, x + 8, x + 16, .. run on XCD x % 8, and they get
  // consecutive logical indices, so that one (b, h)'s blocks share an XCD
  const int nblk = gridDim.x;
  const int xcd = blockIdx.x & 7;
  const int logical = xcd * (nblk >> 3) + min(xcd, nblk & 7) + (blockIdx.x >> 3);
  const int gblocks = (geo.NG + TK_GROUPS - 1) / TK_GROUPS;
  const int slot = logical / gblocks;
  const int gblock = logical - slot * gblocks;
  const int b = slot / geo.H;
  const int h = geo.order[slot - b * geo.H];
  const int bh = b * geo.H + h;
  const int S = geo.S;
  const int kh = geo.k[h];
  const long long head_base = (long long)bh * S * R;   // element offset of (b,h) in Q_lr/K_lr

  const unsigned char* klr = static_cast<const unsigned char*>(klr_) + head_base * C::ES;
  const unsigned char* qlr = static_cast<const unsigned char*>(qlr_) + head_base * C::ES;

  // ---- group state
  for (int i = tid; i < TK_GROUPS; i += TK_THREADS) {
    st_prefix[i] = 0;
    st_krem[i] = kh;
    st_npass[i] = (gblock * TK_GROUPS + i < geo.NG) ? 0 : -1;   // -1: no such group
  }
  for (int i = tid; i < TK_GROUPS * TK_HSTRIDE; i += TK_THREADS) hist[i] = 0;

  // ---- group sums -> A operands (row li = group 16*gw + li); each key slice sums its own copy
  const GroupGeom gg{geo.Hh, geo.W, geo.gt, geo.gh, geo.gw, geo.nbh, geo.nbw};
  const int my_group = gblock * TK_GROUPS + 16 * gw + li;
  float ssum[C::KSTEPS * (F32 ? 1 : 8)];
#pragma unroll
  for (int i = 0; i < C::KSTEPS * (F32 ? 1 : 8); ++i) ssum[i] = 0.0f;
  if (my_group < geo.NG) {
    for (int j = 0; j < geo.G; ++j) {
      const int n = gg.token(my_group, j);
      const unsigned char* row = qlr + (long long)n * C::RB;
      if constexpr (F32) {
        const float* fr = reinterpret_cast<const float*>(row) + lg * (R / 4);
#pragma unroll
        for (int s = 0; s < R / 4; ++s) ssum[s] += fr[s];
      } else {
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
          if (ks * 32 + 8 * lg < R) {
            const u32x4 v = ld16(row + (ks * 32 + 8 * lg) * 2);
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
              ssum[ks * 8 + 2 * e2] += bf16_lo(v[e2]);
              ssum[ks * 8 + 2 * e2 + 1] += bf16_hi(v[e2]);
            }
          }
        }
      }
    }
  }
  // bf16 path: s = hi + lo with hi = bf16(s), lo = bf16(s - hi); exact while |s| < 2^16 for
  // integer sums, and products with bf16 K_lr entries are exact in the fp32 accumulator.
  u32x4 a_hi[F32 ? 1 : C::KSTEPS], a_lo[F32 ? 1 : C::KSTEPS];
  if constexpr (!F32) {
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float s0 = ssum[ks * 8 + 2 * e2], s1 = ssum[ks * 8 + 2 * e2 + 1];
        const float h0 = bf16_round(s0), h1 = bf16_round(s1);
        a_hi[ks][e2] = pack_bf16(h0, h1);
        a_lo[ks][e2] = pack_bf16(s0 - h0, s1 - h1);
      }
    }
  }

  // ---- B operands: key m = TK_TILE t + 16 kw + li of tile t (clamped to the last key; the
  // scores of keys past the end are never counted), contraction slot lg
  constexpr int NB = F32 ? R / 16 : C::KSTEPS;   // 16-byte loads per lane and tile
  auto load_b = [&](int t, u32x4* bo) {
    const int m = min(t * TK_TILE + 16 * kw + li, S - 1);
    const unsigned char* krow = klr + (long long)m * C::RB;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if constexpr (F32) {
        bo[i] = ld16(krow + (lg * (R / 4) + 4 * i) * 4);
      } else {
        bo[i] = (i * 32 + 8 * lg < R) ? ld16(krow + (i * 32 + 8 * lg) * 2) : u32x4{0, 0, 0, 0};
      }
    }
  };
  // scores of the wave's 16 groups (rows 4 lg + j) against its key of the tile (column li)
  auto scores = [&](const u32x4* bo) -> floatx4 {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(ssum[4 * i + e], __uint_as_float(bo[i][e]), acc);
      } else {
        acc = mfma_bf16(a_hi[i], bo[i], acc);
        acc = mfma_bf16(a_lo[i], bo[i], acc);
      }
    }
    return acc;
  };
  const int ntiles = (S + TK_TILE - 1) / TK_TILE;

  __syncthreads();

  // ---- radix passes (pass 4 = compaction)
  for (int pass = 0; pass <= 4; ++pass) {
    if (pass < 4) {
      if (tid == 0) {
        int act = 0;
        for (int i = 0; i < TK_GROUPS; ++i) act |= (st_npass[i] == pass);
        st_active[pass] = act;
      }
      __syncthreads();
      if (!st_active[pass]) continue;   // uniform: every group stopped refining earlier
    }
    const int dshift = 24 - 8 * pass;
    const int pshift = 32 - 8 * pass;
    u32x4 bcur[NB], bnxt[NB];
    load_b(0, bcur);
    if (pass < 4) {
      // Histogram pass. Slot j of lane li is group 4 lg + (j + li) % 4 of the wave's block.
      uint32_t rpfx[4];
      int rstate[4];
      uint32_t* rhist[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gl = 16 * gw + 4 * lg + ((j + li) & 3);
        rpfx[j] = st_prefix[gl];
        rstate[j] = st_npass[gl];
        rhist[j] = &hist[gl * TK_HSTRIDE];
      }
      for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) load_b(t + 1, bnxt);
        const floatx4 acc = scores(bcur);
        const bool mvalid = t * TK_TILE + 16 * kw + li < S;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int jr = (j + li) & 3;
          const float sc = jr == 0 ? acc[0] : jr == 1 ? acc[1] : jr == 2 ? acc[2] : acc[3];
          const uint32_t key = score_key(sc);
          const bool take = mvalid && rstate[j] == pass &&
                            (pass == 0 || (key >> (pshift & 31)) == rpfx[j]);
          if (take)
            __hip_atomic_fetch_add(&rhist[j][(key >> dshift) & 255u], 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) bcur[i] = bnxt[i];
      }
    } else {
      // Compaction. Lane: key m, groups 4 lg + j of the wave's block, all finished.
      uint32_t pfx[4];
      int shift[4], cnt[4], left[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gl = 16 * gw + 4 * lg + j;
        const int gs = st_npass[gl];
        pfx[j] = gs >= 16 ? st_prefix[gl] : 0xffffffffu;
        shift[j] = gs >= 16 ? 32 - 8 * (gs - 16) : 0;   // no key exceeds an all-ones image
        left[j] = gs >= 16 ? st_krem[gl] : 0;            // equal keys still to take
        cnt[j] = 0;
      }
      // rows of groups 4 lg + j are consecutive (k_h entries each); groups past NG select nothing
      int32_t* const orow = idx + geo.row_offset(b, h, gblock * TK_GROUPS + 16 * gw + 4 * lg);
      const uint32_t below = (1u << li) - 1u;
      for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) load_b(t + 1, bnxt);
        const floatx4 acc = scores(bcur);
        const int m = t * TK_TILE + 16 * kw + li;
        const bool mvalid = m < S;
        uint32_t ge[4];   // this slice's ballots of the key's group j: above (bits 0..15), equal
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t v = score_key(acc[j]) >> (shift[j] & 31);
          const uint32_t gtb = (uint32_t)(__ballot(mvalid && v > pfx[j]) >> (16 * lg)) & 0xffffu;
          const uint32_t eqb = (uint32_t)(__ballot(mvalid && v == pfx[j]) >> (16 * lg)) & 0xffffu;
          ge[j] = gtb | (eqb << 16);
          if (li == 0)
            tcnt[t & 1][16 * gw + 4 * lg + j][kw] = __popc(gtb) | (__popc(eqb) << 16);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 c = *reinterpret_cast<const u32x4*>(&tcnt[t & 1][16 * gw + 4 * lg + j][0]);
          uint32_t pre = 0, tot = 0;   // (above, equal) counts of the earlier slices / all slices
#pragma unroll
          for (int w = 0; w < TK_KW; ++w) {
            if (w < kw) pre += c[w];
            tot += c[w];
          }
          const int pre_gt = (int)(pre & 0xffffu), pre_eq = (int)(pre >> 16);
          const int lft = max(left[j], 0);
          const bool sel = ((ge[j] >> li) & 1u) ||
                           (((ge[j] >> (16 + li)) & 1u) &&
                            pre_eq + __popc((ge[j] >> 16) & below) < lft);
          const uint32_t selbits = (uint32_t)(__ballot(sel) >> (16 * lg)) & 0xffffu;
          const int pos = cnt[j] + pre_gt + min(lft, pre_eq) + __popc(selbits & below);
          if (sel && pos < kh) orow[j * kh + pos] = m;
          cnt[j] += (int)(tot & 0xffffu) + min(lft, (int)(tot >> 16));
          left[j] -= (int)(tot >> 16);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) bcur[i] = bnxt[i];
      }
    }

    if (pass < 4) {
      __syncthreads();
      // Each wave resolves digit `pass` for some of the groups and clears their histograms.
      for (int gl = wave; gl < TK_GROUPS; gl += TK_WAVES) {
        if (st_npass[gl] != pass) continue;   // uniform across the wave
        uint32_t* hrow = &hist[gl * TK_HSTRIDE];
        uint32_t c[4];
        uint32_t lsum = 0;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          c[tt] = hrow[255 - (4 * lane + tt)];
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
        if (excl < krem && krem <= incl) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            if (excl + c[tt] >= krem) {
              const uint32_t bin = 255u - (4u * lane + tt);
              const uint32_t left = krem - excl;   // keys still needed inside `bin`
              st_prefix[gl] = (pass == 0) ? bin : ((st_prefix[gl] << 8) | bin);
              st_krem[gl] = (int)left;
              st_npass[gl] = (left == c[tt] || pass == 3) ? 16 + pass + 1 : pass + 1;
              break;
            }
            excl += c[tt];
          }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) hrow[4 * lane + tt] = 0;
      }
      __syncthreads();
    }
  }
}

}  // namespace

int launch_topk(const Geom& geo, const void* q_lr, const void* k_lr, int32_t* idx, void* stream) {
  const int gblocks = (geo.NG + TK_GROUPS - 1) / TK_GROUPS;
  const dim3 grid(geo.B * geo.H * gblocks);
  const dim3 block(TK_THREADS);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool f32 = geo.dtype == DSV_FP32;
#define DSV_TOPK_CASE(F, RR)                                                               \
  if (f32 == F && geo.r == RR) {                                                           \
    hipLaunchKernelGGL((topk_kernel<F, RR>), grid, block, 0, st, q_lr, k_lr, idx, geo);    \
    return (int)hipGetLastError();                                                         \
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
