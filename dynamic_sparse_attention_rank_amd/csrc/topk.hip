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
//   * Workgroup = 4 waves = 64 groups of one (b, h). Each wave owns 16 groups: the 16-row A
//     operand of a v_mfma_f32_16x16x32_bf16 holds their group sums (split into two bf16 terms,
//     hi + lo, so that the sums stay exact), the B operand holds 16 keys of K_lr staged in LDS.
//     Each 16x16 output tile gives a lane one key and four groups.
//   * Exact selection = radix select on an order-preserving 32-bit image of the fp32 score,
//     8 bits per pass: pass p builds, per group, an LDS histogram of digit p over the keys whose
//     higher digits match the prefix found so far; a wave scan then fixes the digit holding the
//     k-th largest key. A group stops refining as soon as its whole current bin is needed.
//   * A final pass compacts, per group, the keys above the threshold plus the first `need` keys
//     equal to it, in ascending key order (wave ballots give each lane its output slot).
//   * K_lr tiles are staged once per workgroup in LDS (double-buffered) and read by all waves.
#include "device_common.h"
#include "dsv_internal.h"

namespace dsv {
namespace {

constexpr int TK_WAVES = 4;
constexpr int TK_THREADS = 64 * TK_WAVES;
constexpr int TK_GROUPS = 16 * TK_WAVES;   // groups per workgroup
constexpr int TK_TILE = 64;                // keys per staged K_lr tile
constexpr int TK_HSTRIDE = 257;            // 256 bins + 1 pad word per group histogram

// Order-preserving map float -> uint32 (larger score <=> larger key). -0 is folded onto +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  if (s == 0.0f) s = 0.0f;
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <bool F32, int R>
struct TopkCfg {
  static constexpr int ES = F32 ? 4 : 2;             // bytes per element
  static constexpr int RB = R * ES;                  // bytes per K_lr row
  static constexpr int TILE_BYTES = TK_TILE * RB;
  static constexpr int CHUNKS = TILE_BYTES / 16;     // 16-byte chunks per tile
  static constexpr int LD_PER_THREAD = (CHUNKS + TK_THREADS - 1) / TK_THREADS;
  static constexpr int KSTEPS = F32 ? R / 4 : (R + 31) / 32;   // MFMA contraction steps
};

template <bool F32, int R>
__global__ __launch_bounds__(TK_THREADS) void topk_kernel(const void* __restrict__ qlr_,
                                                          const void* __restrict__ klr_,
                                                          int32_t* __restrict__ idx, Geom geo) {
  using C = TopkCfg<F32, R>;
  __shared__ uint32_t hist[TK_GROUPS * TK_HSTRIDE];
  __shared__ __attribute__((aligned(16))) unsigned char ktile[2][C::TILE_BYTES];
  __shared__ uint32_t st_prefix[TK_GROUPS];
  __shared__ int st_krem[TK_GROUPS];
  // Group state: -1 = no such group; 0..3 = still refining, that many digits known (and the
  // next histogram pass is that index); 16 + D = finished with D digits known.
  __shared__ int st_npass[TK_GROUPS];
  __shared__ int st_active;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lg = lane >> 4;
  const int li = lane & 15;

  const int gblocks = (geo.NG + TK_GROUPS - 1) / TK_GROUPS;
  const int bh = blockIdx.x / gblocks;
  const int gblock = blockIdx.x - bh * gblocks;
  const int b = bh / geo.H;
  const int h = bh - b * geo.H;
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

  // ---- group sums -> A operands (row li = group 16*wave + li)
  const GroupGeom gg{geo.Hh, geo.W, geo.gt, geo.gh, geo.gw, geo.nbh, geo.nbw};
  const int my_group = gblock * TK_GROUPS + 16 * wave + li;
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

  // ---- K_lr tile staging
  const int ntiles = (S + TK_TILE - 1) / TK_TILE;
  auto load_tile = [&](int t, u32x4* regs) {
#pragma unroll
    for (int c = 0; c < C::LD_PER_THREAD; ++c) {
      const int chunk = tid + c * TK_THREADS;
      regs[c] = u32x4{0, 0, 0, 0};
      if (chunk < C::CHUNKS) {
        const long long byte = (long long)t * C::TILE_BYTES + chunk * 16;
        const int key = (int)(byte / C::RB);
        if (key < S) regs[c] = ld16(klr + byte);
      }
    }
  };
  auto store_tile = [&](int buf, const u32x4* regs) {
#pragma unroll
    for (int c = 0; c < C::LD_PER_THREAD; ++c) {
      const int chunk = tid + c * TK_THREADS;
      if (chunk < C::CHUNKS) *reinterpret_cast<u32x4*>(&ktile[buf][chunk * 16]) = regs[c];
    }
  };

  // Scores of the 16 keys of sub-tile `sub` for this wave's 16 groups (lane: key li, rows 4lg+j).
  auto tile_scores = [&](int buf, int sub) -> floatx4 {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    const unsigned char* krow = &ktile[buf][(sub * 16 + li) * C::RB];
    if constexpr (F32) {
      const float* kr = reinterpret_cast<const float*>(krow) + lg * (R / 4);
#pragma unroll
      for (int s = 0; s < R / 4; ++s) acc = mfma_f32(ssum[s], kr[s], acc);
    } else {
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        u32x4 bop = {0, 0, 0, 0};
        if (ks * 32 + 8 * lg < R) bop = *reinterpret_cast<const u32x4*>(krow + (ks * 32 + 8 * lg) * 2);
        acc = mfma_bf16(a_hi[ks], bop, acc);
        acc = mfma_bf16(a_lo[ks], bop, acc);
      }
    }
    return acc;
  };

  __syncthreads();

  // ---- radix passes (pass 4 = compaction)
  for (int pass = 0; pass <= 4; ++pass) {
    if (pass < 4) {
      if (tid == 0) {
        int act = 0;
        for (int i = 0; i < TK_GROUPS; ++i) act |= (st_npass[i] == pass);
        st_active = act;
      }
      __syncthreads();
      if (!st_active) continue;   // uniform: every group stopped refining earlier
    }
    // per-lane copies of the state of the lane's four groups (rows 4*lg + j of the wave block)
    uint32_t pfx[4];
    int gstate[4], need[4], shift[4];
    long long rowoff[4];
    int cnt[4] = {0, 0, 0, 0}, ties[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gl = 16 * wave + 4 * lg + j;
      pfx[j] = st_prefix[gl];
      gstate[j] = st_npass[gl];
      need[j] = st_krem[gl];
      shift[j] = 32 - 8 * (gstate[j] - 16);   // meaningful once finished (gstate >= 16)
      rowoff[j] = (gstate[j] >= 0) ? geo.row_offset(b, h, gblock * TK_GROUPS + gl) : 0;
    }

    u32x4 regs[C::LD_PER_THREAD];
    load_tile(0, regs);
    store_tile(0, regs);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      if (t + 1 < ntiles) load_tile(t + 1, regs);
      floatx4 accs[TK_TILE / 16];   // all sub-tiles' scores first: the LDS reads and MFMAs
#pragma unroll                     // of the tile overlap instead of waiting one by one
      for (int sub = 0; sub < TK_TILE / 16; ++sub) accs[sub] = tile_scores(buf, sub);
#pragma unroll
      for (int sub = 0; sub < TK_TILE / 16; ++sub) {
        const int m = t * TK_TILE + sub * 16 + li;
        const floatx4 acc = accs[sub];
        const bool mvalid = m < S;
        if (pass < 4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t key = score_key(acc[j]);
            const bool take = mvalid && gstate[j] == pass &&
                              (pass == 0 || (key >> (32 - 8 * pass)) == pfx[j]);
            if (take) {
              const int gl = 16 * wave + 4 * lg + j;
              __hip_atomic_fetch_add(&hist[gl * TK_HSTRIDE + ((key >> (24 - 8 * pass)) & 255u)], 1u,
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
          }
        } else {
          const uint32_t below = (1u << li) - 1u;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t key = score_key(acc[j]);
            const bool gvalid = gstate[j] >= 16;
            const uint32_t v = key >> (shift[j] & 31);
            const bool gt = mvalid && gvalid && v > pfx[j];
            const bool eq = mvalid && gvalid && v == pfx[j];
            const uint32_t eqbits = (uint32_t)(__ballot(eq) >> (16 * lg)) & 0xffffu;
            const bool sel = gt || (eq && ties[j] + __popc(eqbits & below) < need[j]);
            const uint32_t selbits = (uint32_t)(__ballot(sel) >> (16 * lg)) & 0xffffu;
            const int pos = cnt[j] + __popc(selbits & below);
            if (sel && pos < kh) idx[rowoff[j] + pos] = m;
            cnt[j] += __popc(selbits);
            ties[j] += __popc(eqbits);
          }
        }
      }
      if (t + 1 < ntiles) store_tile(buf ^ 1, regs);
      __syncthreads();
    }

    if (pass < 4) {
      // Each wave resolves digit `pass` for its own 16 groups and clears their histograms.
      for (int gi = 0; gi < 16; ++gi) {
        const int gl = 16 * wave + gi;
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
