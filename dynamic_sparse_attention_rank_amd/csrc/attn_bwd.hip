// attn_bwd.hip — query-grouped sparse attention, backward (dQ, dK, dV) with the index lists
// held constant.
//
// The DSV summaries (gist.science/{zh,pt,fr,ko}/paper/2502.07590) report sparse *training*
// throughput (zh §4 / pt §4: up to 3.02x over full attention), which needs the backward of
// the sparse attention of zh §2.1; the pages do not describe it. This is the standard softmax
// attention gradient restricted to each group's selected keys:
//     P = exp(scale q.k - LSE), Delta_n = dO_n . O_n, dS = P * (dO.v - Delta)
//     dQ_n = scale sum_m dS[n,m] k_m     (owned by the group: written once)
//     dK_m = scale sum_n dS[n,m] q_n     (summed over every group that selected m)
//     dV_m = sum_n P[n,m] dO_n           (idem)
//
// bf16 path (gfx950 MFMA), one wave per group, keys in chunks of 32:
//   * Q and dO rows of the group sit in LDS (one swizzled copy each). S = Q K^T and
//     dP = dO V^T read them as 16-byte A operands, with K / V rows gathered straight into B
//     operands; a lane then holds one key and 4 queries per 16x16 tile, which is exactly the
//     B operand of dV^T = dO^T P and dK^T = Q^T dS. Their A operands (dO, Q with queries
//     contiguous per lane) are transposed LDS reads (ds_read_b64_tr_b16).
//   * dQ^T += K^T dS^T: K^T from the K registers by an MFMA against a 0/1 selection operand,
//     dS^T from a [key][member] LDS tile read back transposed. dQ is written once.
//   * dK/dV: each (group, selected key) edge yields one row of dV and one of dK, summed over
//     all groups that selected the key. fp32 atomics on this chip sustain only ~0.33 T adds/s,
//     so the rows are not added in place. The edge (g, p) owns staging row g*padded_k + p.
//     Per (tensor, 16-key block) the block's largest entry m chooses the format: at d = 128
//     with m <= kStage8Bound, 8-bit codes scaled by m (absolute error <= m/254 <= 5e-4 per
//     entry); else fp16 times a power of two (relative error <= 2^-11). The rows are written
//     with whole-line non-temporal stores, one factor per block to a small table that the
//     reduce reads through L2.
//     Small pre-passes list, for every 32-key bucket, its edges ordered by key, then by
//     group; a reduce kernel then sums each key's rows in registers (one wave per bucket and
//     tensor, one row per load instruction, no atomics, no LDS) and writes every dK/dV row
//     exactly once, so dK/dV are bitwise reproducible. Heads are processed in chunks sized to
//     the caller's workspace.
// fp32 path: v_mfma_f32_16x16x4_f32 tiles, one wave per group, 16-key chunks through LDS;
// dK/dV are summed as 2^-32 fixed-point 64-bit integers (order-independent, so reproducible
// bit for bit). It exists for fp32 inputs and is not tuned for speed.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "dsv_internal.h"

namespace dsv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void decode_unit(const Geom& geo, int unit, int& b, int& h, int& g) {
  const int per_head = geo.B * geo.NG;
  const int slot = unit / per_head;
  const int rem = unit - slot * per_head;
  h = geo.order[slot];
  b = rem / geo.NG;
  g = rem - b * geo.NG;
}


// 32 keys per dK/dV bucket: a bucket's key offset fits the 5 low bits of a list entry, and
// its keys' rows form one list that one reduce wave per tensor walks
constexpr int kBucketLog2 = 5;
constexpr int kBucket = 1 << kBucketLog2;
constexpr int kMaxChunk = 64;    // (b, h) slots per chunk
constexpr int kPermWaves = 4;    // waves per bucket in the edge-list placement
// fp16 staging rows are the entries times one power-of-two scale per (group, 16-key block):
// kStageMax / m (m the block's largest |entry|) rounded down to a power of two keeps every
// scaled entry within kStageMax (fp16 reaches 65504), and fp16's 11-bit significand gives each
// entry a relative error <= 2^-11 whatever its size, down to 2^-28 of m where fp16 turns
// subnormal.
constexpr float kStageMax = 16384.f;
// Blocks whose largest |entry| m (in true units) is within kStage8Bound are staged as 8-bit
// rows (d = 128): code = 128 + round(x * 127 / m), so every entry is off by at most
// m/254 <= kStage8Bound/254 ~ 5e-4, and a row takes half the bytes of fp16. (At 0.5 the worst
// dK/dV error over the 20 Training steps reached 82% of the 2e-2 bar: a key's sum carries the
// errors of some 50 groups' rows.)
constexpr float kStage8Bound = 0.125f;
template <int D>
constexpr bool kStage8 = D == 128;

// kStageMax / bound rounded down to a power of two (clamped to [2^-126, 2^100]); 0 if bound
// is not positive (the block is all zero).
__device__ __forceinline__ float pow2_scale(float bound) {
  if (!(bound > 0.f)) return 0.f;
  const float x =
      fminf(fmaxf(kStageMax * __builtin_amdgcn_rcpf(bound), 1.17549435e-38f), 1.2676506e30f);
  return __uint_as_float(__float_as_uint(x) & 0xff800000u);
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 v;
  v.x = (_Float16)lo;
  v.y = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

__host__ __device__ inline int n_buckets(int S) { return (S + kBucket - 1) / kBucket; }

// Staging rows per group: k rounded up to the 32-key chunk, so that the backward kernel's
// stores are unconditional (the tail rows of a group hold zeros and are never read).
__host__ __device__ inline int padded_k(int k) { return (k + 31) & ~31; }

// A chunk of consecutive (b, h) slots in launch order (slot s = head rank * B + b).
struct Chunk {
  int s0, n;
  long long edge_base[kMaxChunk + 1];   // first buffer row of each slot; [n] = rows in chunk
};

__device__ __forceinline__ void chunk_slot(const Geom& geo, int s, int& b, int& h) {
  const int hs = s / geo.B;
  b = s - hs * geo.B;
  h = geo.order[hs];
}

// Row entry points: rs[g][j] = first position of row g whose key lies in bucket >= j
// (rs[g][nB] = k). One wave per row; rows are ascending, so each bucket's keys form one run.
// Position p writes the buckets after its predecessor's, up to its own; the lanes load eight
// 64-key steps of the row at once, and a step's predecessor buckets come from the lane below
// (lane 0: the previous step's lane 63).
__global__ __launch_bounds__(256) void row_bucket_starts(const int32_t* __restrict__ idx, Chunk ch,
                                                         uint32_t* __restrict__ rs, Geom geo) {
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (wave >= ch.n * geo.NG) return;
  const int sl = wave / geo.NG;
  const int g = wave - sl * geo.NG;
  int b, h;
  chunk_slot(geo, ch.s0 + sl, b, h);
  const int kh = geo.k[h];
  const int nB = n_buckets(geo.S);
  const int32_t* row = idx + geo.row_offset(b, h, g);
  uint32_t* r = rs + (long long)wave * (nB + 1);
  int prev = -1;   // bucket of the key before the step's first
  for (int p0 = 0; p0 < kh; p0 += 8 * 64) {
    int kv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) kv[u] = row[min(p0 + 64 * u + lane, kh - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + 64 * u + lane;
      const int jp = clamp_key(kv[u], geo.S) >> kBucketLog2;
      const int below = __shfl_up(jp, 1, 64);
      const int jq = lane == 0 ? prev : below;
      prev = __shfl(jp, 63, 64);
      if (p < kh)
        for (int j = jq + 1; j <= jp; ++j) r[j] = (uint32_t)p;
    }
  }
  const int jl = clamp_key(row[kh - 1], geo.S) >> kBucketLog2;
  for (int j = jl + 1 + lane; j <= nB; j += 64) r[j] = (uint32_t)kh;
}

// rs [slot][g][j] -> rsT [slot][j][g] through 64 x 64 LDS tiles, so that the per-bucket
// passes below read a bucket's entry points of consecutive groups from consecutive words.
__global__ __launch_bounds__(256) void transpose_rs(const uint32_t* __restrict__ rs,
                                                    uint32_t* __restrict__ rsT, Geom geo) {
  __shared__ uint32_t t[64][65];
  const int nB1 = n_buckets(geo.S) + 1;
  const int tj = (nB1 + 63) / 64, tg = (geo.NG + 63) / 64;
  int bid = blockIdx.x;
  const int sl = bid / (tj * tg);
  bid -= sl * tj * tg;
  const int j0 = (bid % tj) * 64, g0 = (bid / tj) * 64;
  const uint32_t* src = rs + (long long)sl * geo.NG * nB1;
  uint32_t* dst = rsT + (long long)sl * geo.NG * nB1;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int g = g0 + r, j = j0 + tx;
    if (g < geo.NG && j < nB1) t[r][tx] = src[(long long)g * nB1 + j];
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int j = j0 + r, g = g0 + tx;
    if (g < geo.NG && j < nB1) dst[(long long)j * geo.NG + g] = t[tx][r];
  }
}

// Row-run length of bucket j in row g: the entry points lie in [0, k] whatever the row holds
// (every j is written), but only an ascending row makes them non-decreasing; a decreasing pair
// counts as an empty run so that a malformed row cannot produce a negative length.
__device__ __forceinline__ uint32_t run_len(uint32_t a, uint32_t b) { return b > a ? b - a : 0u; }

// tot[j] = staging rows whose key lies in bucket j (all groups of the slot). One wave per
// (slot, bucket), lanes over groups; entry points from the transposed table rsT.
__global__ __launch_bounds__(64) void bucket_totals(const uint32_t* __restrict__ rsT,
                                                    uint32_t* __restrict__ tot, Geom geo) {
  const int nB = n_buckets(geo.S);
  const int sl = blockIdx.x / nB;
  const int j = blockIdx.x - sl * nB;
  const uint32_t* r = rsT + (long long)sl * geo.NG * (nB + 1) + (long long)j * geo.NG;
  uint32_t run = 0;
  for (int g = threadIdx.x; g < geo.NG; g += 64) run += run_len(r[g], r[geo.NG + g]);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) run += __shfl_xor(run, m, 64);
  if (threadIdx.x == 0) tot[(long long)sl * (nB + 1) + j] = run;
}

// off[j] = exclusive prefix of tot over buckets (off[nB] = rows of the slot).
__global__ __launch_bounds__(256) void bucket_offsets(const uint32_t* __restrict__ tot,
                                                      uint32_t* __restrict__ off, Geom geo) {
  const int nB = n_buckets(geo.S);
  const uint32_t* c = tot + (long long)blockIdx.x * (nB + 1);
  uint32_t* o = off + (long long)blockIdx.x * (nB + 1);
  __shared__ uint32_t part[256];
  const int per = (nB + 255) / 256;
  const int j0 = threadIdx.x * per;
  uint32_t sum = 0;
  for (int j = j0; j < min(j0 + per, nB); ++j) sum += c[j];
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int stride = 1; stride < 256; stride <<= 1) {
    const uint32_t x = threadIdx.x >= stride ? part[threadIdx.x - stride] : 0u;
    __syncthreads();
    part[threadIdx.x] += x;
    __syncthreads();
  }
  uint32_t run = part[threadIdx.x] - sum;
  for (int j = j0; j < min(j0 + per, nB); ++j) {
    o[j] = run;
    run += c[j];
  }
  if (threadIdx.x == 255) o[nB] = part[255];
}

// Bucket edge list, by key: perm[off[j] + i], i < tot[j], holds the edges (g, p) whose key
// lies in bucket j, ordered by key, then by group, each as (slot-relative staging row
// g*padded_k + p) << 5 | (key - 32 j). kPermWaves waves per (slot, bucket), each over its own
// run of 64-group steps. A lane turns its group's run of keys in the bucket into a mask of key
// offsets (the run ascends, so the run's i-th key sits at staging row e0 + i, i = the number of
// mask bits below it). A first sweep counts each key's groups (one ballot per key) and keeps
// each group's mask and first staging row in LDS (dynamic, 8 bytes per group, when the launch
// provides them); the waves' counts give each key's first list position per wave, and a
// second sweep places every edge after those of the key's earlier groups (ballot and
// lane-prefix count). A 128-byte line of an index row holds the keys of about ten consecutive
// buckets, so the block index is remapped to give each XCD a contiguous range of buckets (one
// L2 then serves a line to all of them).
__global__ __launch_bounds__(64 * kPermWaves) void bucket_perm(
    const uint32_t* __restrict__ rsT, const uint32_t* __restrict__ off,
    const int32_t* __restrict__ idx, Chunk ch, uint32_t* __restrict__ perm, Geom geo, int cached) {
  extern __shared__ uint2 mcache[];   // [NG] {key mask, first staging row} when cached
  __shared__ uint32_t wcnt[kPermWaves][kBucket];   // each wave's edges per key offset
  const int nB = n_buckets(geo.S);
  const int nblk = gridDim.x, xcd = blockIdx.x & 7;
  const int logical = xcd * (nblk >> 3) + min(xcd, nblk & 7) + (blockIdx.x >> 3);
  const int sl = logical / nB;
  const int j = logical - sl * nB;
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  int b, h;
  chunk_slot(geo, ch.s0 + sl, b, h);
  const uint32_t kh = (uint32_t)geo.k[h];
  const uint32_t kp = (uint32_t)padded_k(geo.k[h]);
  const uint32_t slot_rows = (uint32_t)(ch.edge_base[sl + 1] - ch.edge_base[sl]);
  const uint32_t* r = rsT + (long long)sl * geo.NG * (nB + 1) + (long long)j * geo.NG;
  const int32_t* keys = idx + geo.row_offset(b, h, 0);   // row of group g: keys + g*k
  uint32_t* pm = perm + ch.edge_base[sl];
  const int key0 = j * kBucket;
  // the wave's groups: a run of whole 64-group steps, in group order across the waves
  const int nsteps = (geo.NG + 63) / 64;
  const int spw = (nsteps + kPermWaves - 1) / kPermWaves;
  const int gbeg = min(wv * spw, nsteps) * 64, gend = min((wv + 1) * spw, nsteps) * 64;
  // mask of the key offsets of group g0 + lane's run in the bucket; a = the run's first
  // position. A malformed (not ascending) row may repeat an offset: the mask then holds fewer
  // edges than the run, and no more than the list has room for are placed.
  auto run_mask = [&](int g0, uint32_t& a) {
    const int g = g0 + lane;
    uint32_t len = 0;
    a = 0;
    if (g < geo.NG) {
      a = r[g];
      len = run_len(a, r[geo.NG + g]);
    }
    const int32_t* krow = keys + (long long)g * kh + a;
    uint32_t maxlen = len;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) maxlen = max(maxlen, (uint32_t)__shfl_xor((int)maxlen, m, 64));
    uint32_t mask = 0;
    for (uint32_t i0 = 0; i0 < maxlen; i0 += 8) {
      int kv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) kv[u] = i0 + u < len ? krow[i0 + u] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u < len)
          mask |= 1u << min(max(clamp_key(kv[u], geo.S) - key0, 0), kBucket - 1);
    }
    return mask;
  };
  // first sweep: groups per key offset
  uint32_t cnt[kBucket];
#pragma unroll
  for (int ko = 0; ko < kBucket; ++ko) cnt[ko] = 0;
  for (int g0 = gbeg; g0 < gend; g0 += 64) {
    uint32_t a;
    const uint32_t mask = run_mask(g0, a);
    if (cached && g0 + lane < geo.NG)
      mcache[g0 + lane] = make_uint2(mask, (uint32_t)(g0 + lane) * kp + a);
#pragma unroll
    for (int ko = 0; ko < kBucket; ++ko)
      cnt[ko] += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64((mask >> ko) & 1u));
  }
  // first list position of each key offset for this wave: the bucket's offset, the edges of
  // the lower key offsets (all waves), then those of the earlier waves at the same offset
  uint32_t mine = 0;
#pragma unroll
  for (int ko = 0; ko < kBucket; ++ko) mine = lane == ko ? cnt[ko] : mine;
  if (lane < kBucket) wcnt[wv][lane] = mine;
  __syncthreads();
  uint32_t tk = 0, before = 0;
  if (lane < kBucket) {
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) {
      const uint32_t c = wcnt[w][lane];
      tk += c;
      before += w < wv ? c : 0u;
    }
  }
  uint32_t incl = tk;
#pragma unroll
  for (int o = 1; o < kBucket; o <<= 1) {
    const uint32_t x = (uint32_t)__shfl_up((int)incl, o, 64);
    if (lane >= o) incl += x;
  }
  const uint32_t first = off[(long long)sl * (nB + 1) + j] + incl - tk + before;
  uint32_t base[kBucket];   // next list position of each key offset (uniform)
#pragma unroll
  for (int ko = 0; ko < kBucket; ++ko) base[ko] = (uint32_t)__builtin_amdgcn_readlane((int)first, ko);
  // second sweep: place the edges; an edge's staging row is the run's first row plus the
  // number of the run's keys below it
  for (int g0 = gbeg; g0 < gend; g0 += 64) {
    uint32_t mask = 0u, e = 0u;
    if (cached) {   // written by this lane in the first sweep: no barrier needed
      if (g0 + lane < geo.NG) {
        const uint2 c = mcache[g0 + lane];
        mask = c.x;
        e = c.y;
      }
    } else {
      uint32_t a;
      mask = run_mask(g0, a);
      e = (uint32_t)(g0 + lane) * kp + a;
    }
#pragma unroll
    for (int ko = 0; ko < kBucket; ++ko) {
      const uint32_t bit = (mask >> ko) & 1u;
      const uint64_t m = __builtin_amdgcn_ballot_w64(bit != 0u);
      const uint32_t pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, base[ko]));
      // a malformed row is dropped rather than written past the slot's list
      if (bit != 0u && pos < slot_rows) pm[pos] = (e << 5) | (uint32_t)ko;
      e += bit;
      base[ko] += (uint32_t)__builtin_popcountll(m);
    }
  }
}

__global__ void fill_zero(float4* __restrict__ p, long long n4) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Sum each bucket's staging rows. The bucket's list is ordered by key, so each key's rows are
// consecutive: the lanes add them in registers and write the key's row once when the key
// changes; at the end, zero rows for the keys nobody selected. Each block takes 64 list entries (edge
// row, key, block factors: one per lane) in two halves of 32 rows, whose loads are requested
// half a block before they are added (entries two blocks ahead, factors one block ahead). No
// LDS, no atomics: each key's rows are added in group order, so dK/dV are bitwise reproducible.
// A block factor f says its rows' format: sign bit clear, fp16 entries times f; set (d = 128
// only), 8-bit codes c meaning (c - 128) * |f|. For those the lane adds c * |f| and, once per
// row, |f|; the key's row is then sum(c * |f|) - 128 * sum(|f|).
typedef float floatx2 __attribute__((ext_vector_type(2)));

// A block of 64 list entries, one per lane: staging row, key offset, the lane's dV and dK
// factors (lanes past the end of the list: zero, same sign, so that they add nothing) and the
// format mode of the wave's tensor's rows (dV and dK blocks choose their formats apart): all
// fp16 (0), all 8-bit (1), mixed (2); the same in every lane.
struct RBlk {
  uint32_t e;
  int kk, mode;
  float sv, sk;
};
__device__ __forceinline__ RBlk make_rblk(uint32_t ent, float2 st, long long r0, long long s1,
                                          long long nrows, bool pair, int half) {
  const int lane = threadIdx.x;
  RBlk k;
  const int n = (int)std::min<long long>(64, s1 - r0);   // <= 0 past the list: no row counts
  k.e = std::min<uint32_t>(ent >> 5, (uint32_t)(nrows - 1));
  k.kk = (int)(ent & 31u);
  k.sv = lane < n ? st.x : copysignf(0.f, st.x);
  k.sk = lane < n ? st.y : copysignf(0.f, st.y);
  const uint64_t m8 = __builtin_amdgcn_ballot_w64(__float_as_int(half ? k.sk : k.sv) < 0);
  k.mode = !pair || m8 == 0 ? 0 : m8 == ~0ull ? 1 : 2;
  return k;
}

// The reduce's list walk, pipelined in half blocks: the next block's first half
// is requested before this block's second half is added, its second half before the following
// block's first half; entries three blocks ahead, factors two blocks ahead (a factor is a
// scattered 8-byte read whose address comes from its entry). Every load is unconditional
// (positions clamped; after the last block the "next" blocks reread the last rows, unused),
// and the later blocks' entries and factors go out before the first block's rows, as in the
// loop: the compiler's waits for each half then leave the later requests in flight.
// A macro over the kernel's lambdas load_half, add_half (passed to a function, the row words
// would leave registers).
#define DSV_WALK_BUCKET(PAIR)                                                                 \
  if (s1 > s0) {                                                                              \
    auto row_of = [&](uint32_t ent) {                                                         \
      return std::min<uint32_t>(ent >> 5, (uint32_t)(nrows - 1));                             \
    };                                                                                        \
    const uint32_t ent0 = pm[std::min<long long>(s0 + lane, s1 - 1)];                         \
    uint32_t ent1 = pm[std::min<long long>(s0 + 64 + lane, s1 - 1)];                          \
    const float2 st0 = bfac[(eb + row_of(ent0)) >> 4];                                        \
    uint32_t ent2 = pm[std::min<long long>(s0 + 128 + lane, s1 - 1)];                         \
    float2 st1 = bfac[(eb + row_of(ent1)) >> 4];                                              \
    RBlk cur_b = make_rblk(ent0, st0, s0, s1, nrows, PAIR, half);                             \
    load_half(cur_b, 0);                                                                      \
    load_half(cur_b, 1);                                                                      \
    for (long long r0 = s0; r0 < s1; r0 += 64) {                                              \
      const float2 st2 = bfac[(eb + row_of(ent2)) >> 4];                                      \
      const uint32_t ent3 = pm[std::min<long long>(r0 + 192 + lane, s1 - 1)];                 \
      add_half(cur_b, 0);                                                                     \
      const RBlk nxt = make_rblk(ent1, st1, r0 + 64, s1, nrows, PAIR, half);                  \
      load_half(nxt, 0);                                                                      \
      add_half(cur_b, 1);                                                                     \
      load_half(nxt, 1);                                                                      \
      cur_b = nxt;                                                                            \
      ent1 = ent2;                                                                            \
      st1 = st2;                                                                              \
      ent2 = ent3;                                                                            \
    }                                                                                         \
  }

// One wave per (slot, bucket, half), half 0 = dV, 1 = dK. Lane l owns FPL = d/64 features of
// the half and loads them from each row: d = 128: features 16w + 4g + 2(l%2) + {0,1} with
// g = l/16, w = (l/2)%8, i.e. bytes 2l, 2l + 1 of an 8-bit row (byte 32g + 4w + j <-> feature
// 16w + 4g + j) and fp16 positions 32(w/2) + 8g + 4(w%2) + 2(l%2) + {0,1}. d = 64 (fp16 rows
// only): position l, holding feature 32fp + 4lg + t (t < 4) or 32fp + 16 + 4lg + t - 4 of
// position 32fp + 8lg + t. Both kinds of row sit at the start of the row's 2d-byte place.
template <int D>
__global__ __launch_bounds__(64) void bucket_reduce(const uint32_t* __restrict__ off,
                                                   const uint32_t* __restrict__ perm,
                                                   const float2* __restrict__ bfac,
                                                   const uint16_t* __restrict__ cv,
                                                   const uint16_t* __restrict__ ck, Chunk ch,
                                                   float* __restrict__ dk, float* __restrict__ dv,
                                                   Geom geo) {
  constexpr int FPL = D / 64;   // features per lane
  const int nB = n_buckets(geo.S);
  const int half = blockIdx.x & 1;
  const int bj = blockIdx.x >> 1;
  const int sl = bj / nB;
  const int j = bj - sl * nB;
  const int lane = threadIdx.x;
  int b, h;
  chunk_slot(geo, ch.s0 + sl, b, h);
  const long long bh = (long long)b * geo.H + h;
  const long long eb = ch.edge_base[sl];
  const long long nrows = ch.edge_base[sl + 1] - eb;
  const uint32_t* o = off + (long long)sl * (nB + 1);
  const long long s0 = std::min<long long>(o[j], nrows);
  const long long s1 = std::min<long long>(std::max<long long>(o[j + 1], o[j]), nrows);
  const unsigned char* src =
      reinterpret_cast<const unsigned char*>(half ? ck : cv) + eb * (2 * D);
  const int key0 = j * kBucket;
  const int nk = min(kBucket, geo.S - key0);
  int feat, o16;
  if constexpr (kStage8<D>) {
    const int g = lane >> 4, w = (lane >> 1) & 7, j0 = 2 * (lane & 1);
    feat = 16 * w + 4 * g + j0;
    o16 = 2 * (32 * (w >> 1) + 8 * g + 4 * (w & 1) + j0);
  } else {
    const int t8 = lane & 7;
    feat = (lane & ~31) + 4 * ((lane >> 3) & 3) + (t8 < 4 ? t8 : 12 + t8);
    o16 = 2 * lane;
  }
  const int o8 = 4 * (lane >> 1), sh8 = 16 * (lane & 1);
  float* out = (half ? dk : dv) + bh * geo.S * D + (long long)key0 * D + feat;
  float a0 = 0.f, a1 = 0.f, corr = 0.f;
  int cur = -1;          // key being summed (uniform)
  uint32_t done = 0u;    // keys whose row is written (uniform)
  auto put = [&](int key, float v0, float v1) {
    if constexpr (FPL == 2)
      __builtin_nontemporal_store(floatx2{v0, v1}, reinterpret_cast<floatx2*>(out + key * D));
    else
      out[key * D] = v0;
  };
  // write the finished key (keys nobody selected are zeroed at the end)
  auto close_key = [&]() {
    if (cur >= 0 && cur < nk) {
      put(cur, fmaf(-128.f, corr, a0), fmaf(-128.f, corr, a1));
      done |= 1u << cur;
    }
    a0 = a1 = corr = 0.f;
  };
  using M0 = std::integral_constant<int, 0>;
  using M1 = std::integral_constant<int, 1>;
  using M2 = std::integral_constant<int, 2>;
  uint32_t x[2][32];   // row words of the two halves of a block
  auto load_half = [&](const RBlk& k, int hf) {
    const float sc = half ? k.sk : k.sv;
    auto go = [&](auto mc) {
      constexpr int MODE = decltype(mc)::value;
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        const int u = 32 * hf + v;
        const unsigned char* rp = src + (long long)__builtin_amdgcn_readlane(k.e, u) * (2 * D);
        // staging rows are read once: non-temporal, so they do not displace other lines
        if constexpr (FPL == 1) {
          x[hf][v] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(rp + o16));
        } else if constexpr (MODE == 1) {   // the lane's two codes
          x[hf][v] =
              __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(rp + 2 * lane));
        } else {
          int ob = o16;
          if constexpr (MODE == 2)   // word lane/2 of an 8-bit row
            if (__builtin_amdgcn_readlane(__float_as_int(sc), u) < 0) ob = o8;
          x[hf][v] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(rp + ob));
        }
      }
    };
    if (k.mode == 1) go(M1{});
    else if (k.mode == 0) go(M0{});
    else go(M2{});
  };
  auto add_half = [&](const RBlk& k, int hf) {
    const float sc = half ? k.sk : k.sv;
    auto go = [&](auto mc) {
      constexpr int MODE = decltype(mc)::value;
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        const int u = 32 * hf + v;
        const int ku = __builtin_amdgcn_readlane(k.kk, u);
        const float su = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), u));
        if (ku != cur) {
          close_key();
          cur = ku;
        }
        const uint32_t xv = x[hf][v];
        if constexpr (FPL == 1) {
          a0 = fmaf(su, f16_lo(xv), a0);
        } else if (MODE == 1 || (MODE == 2 && __float_as_int(su) < 0)) {
          const uint32_t w = MODE == 1 ? xv : xv >> sh8;
          a0 = fmaf((float)(w & 0xffu), -su, a0);
          a1 = fmaf((float)((w >> 8) & 0xffu), -su, a1);
          corr -= su;
        } else {
          a0 = fmaf(su, f16_lo(xv), a0);
          a1 = fmaf(su, f16_hi(xv), a1);
        }
      }
    };
    if (k.mode == 1) go(M1{});
    else if (k.mode == 0) go(M0{});
    else go(M2{});
  };
  const uint32_t* pm = perm + eb;
  DSV_WALK_BUCKET(kStage8<D>)
  close_key();
  // zero rows for the keys nobody selected
  for (int key = 0; key < nk; ++key)
    if (!((done >> key) & 1u)) put(key, 0.f, 0.f);
}
#undef DSV_WALK_BUCKET

// LDS copy of the group's Q and dO rows (bf16, [member][feature]). Chunk c (8 features,
// 16 bytes) of row r is stored at chunk position c ^ (r mod D/8): the 16-byte reads of the
// S / dP operands (16 rows, one chunk) then hit distinct banks, and the transposed 8-byte
// reads of ds_read_b64_tr_b16 stay inside one chunk. Rows past the group size are zero.
template <int D>
struct BwdLds {
  uint16_t qn[64 * D];
  uint16_t dn[64 * D];
  uint16_t ds[32 * 80];   // dS tile [key][member], 64 members + 16 pad per row (160 bytes)
  float lse2[64] __attribute__((aligned(16)));    // LSE * log2(e) per group member
  float delta[64] __attribute__((aligned(16)));   // Delta per group member
};

template <int D, int QB>
__global__ __launch_bounds__(64) void attn_bwd_bf16(
    const uint16_t* __restrict__ q, const uint16_t* k,   // k, v: not restrict, so that the
    const uint16_t* v, const uint16_t* __restrict__ o,   // prefetch stays ordered (see below)
    const uint16_t* __restrict__ d_o, const float* __restrict__ lse,
    const int32_t* __restrict__ idx, float scale, float* __restrict__ dq, Chunk ch,
    uint16_t* __restrict__ cv, uint16_t* __restrict__ ck, float2* __restrict__ bfac, Geom geo) {
  constexpr int QBP = (QB + 1) & ~1;   // query blocks padded to whole 32-query k-steps
  constexpr int NM = QBP / 2;
  constexpr int KS = D / 32;
  constexpr int NDB = D / 16;
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  using L = BwdLds<D>;
  __shared__ __attribute__((aligned(16))) L lds;

  const int lane = threadIdx.x;
  const int lg = lane >> 4;
  const int li = lane & 15;
  const int sl = blockIdx.x / geo.NG;   // (b, h) slot inside this chunk
  const int g = blockIdx.x - sl * geo.NG;
  int b, h;
  chunk_slot(geo, ch.s0 + sl, b, h);
  const int kh = geo.k[h];
  const long long bh = (long long)b * geo.H + h;
  const long long base = bh * geo.S * D;
  const uint16_t* Q = q + base;
  const uint16_t* K = k + base;
  const uint16_t* V = v + base;
  const int32_t* row = idx + geo.row_offset(b, h, g);
  const GroupGeom gg{geo.Hh, geo.W, geo.gt, geo.gh, geo.gw, geo.nbh, geo.nbw};
  const int G = geo.G;
  // staging row of edge (g, p): the slot's first row + g*padded_k + p (index order)
  const long long grow = ch.edge_base[sl] + (long long)g * padded_k(kh);

  // ---- per-group set-up: Q and dO rows into LDS, Delta = dO.O and LSE. CPR lanes per row,
  // one chunk each.
  {
    const int rr = lane / CPR, c = lane % CPR;
    for (int r0 = 0; r0 < 16 * QBP; r0 += 64 / CPR) {
      const int r = r0 + rr;
      u32x4 qv = {0u, 0u, 0u, 0u}, dv4 = qv;
      float dacc = 0.f;
      int n = 0;
      if (r < G) {
        n = gg.token(g, r);
        qv = ld16(Q + (long long)n * D + 8 * c);
        dv4 = ld16(d_o + base + (long long)n * D + 8 * c);
        const u32x4 ov = ld16(o + base + (long long)n * D + 8 * c);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          dacc = fmaf(bf16_lo(dv4[w]), bf16_lo(ov[w]), dacc);
          dacc = fmaf(bf16_hi(dv4[w]), bf16_hi(ov[w]), dacc);
        }
      }
      *reinterpret_cast<u32x4*>(&lds.qn[swz<D>(r, 8 * c)]) = qv;
      *reinterpret_cast<u32x4*>(&lds.dn[swz<D>(r, 8 * c)]) = dv4;
#pragma unroll
      for (int m = 1; m < CPR; m <<= 1) dacc += __shfl_xor(dacc, m, 64);
      if (c == 0) {   // padded members: no contribution (P = 0 through lse2 = +inf)
        lds.delta[r] = r < G ? dacc : 0.f;
        lds.lse2[r] = r < G ? lse[bh * geo.S + n] * kLog2e : INFINITY;
      }
    }
  }
  __syncthreads();

  floatx4 dqacc[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int f = 0; f < NDB; ++f) dqacc[qb][f] = floatx4{0.f, 0.f, 0.f, 0.f};
  const float c2 = scale * kLog2e;

  // Every global access in the chunk loop below is unconditional (positions are clamped, tail
  // rows are padding): with gfx9's single in-order vmcnt, a conditional store would force the
  // wait for the prefetched K/V rows to drain every store as well.
  u32x4 kb_n[2][KS], vb_n[2][KS];   // natural K / V rows (B operands) of the current chunk
  int nkey[2];                      // keys of the chunk after the prefetched one
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

  u32x4 sel[2];
  make_selection(lane, sel);

  // One 32-key chunk. The first chunk runs before the loop (peeled) so that both paths into
  // the loop end with the same prefetch-then-store sequence: the compiler's wait for the
  // prefetched K/V rows at the top of the loop then leaves the previous chunk's stores in
  // flight instead of draining them.
  auto chunk = [&](const int cb, auto tail_tag) {
    constexpr bool kTail = decltype(tail_tag)::value;   // keys past the row end in it
    // ---- S = Q K^T, dP = dO V^T of 16-key block kb; lane: key 16kb + li, members 16qb +
    // 4lg + j. The A operands (member 16qb + li, features 32ks + 8lg ..) are 16-byte LDS row
    // reads.
    auto s_dp = [&](const int kb, floatx4 (&s)[QB], floatx4 (&dp)[QB]) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        s[qb] = dp[qb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int off = swz<D>(qb * 16 + li, 32 * ks + 8 * lg);
          s[qb] = mfma_bf16(*reinterpret_cast<const u32x4*>(&lds.qn[off]), kb_n[kb][ks], s[qb]);
          dp[qb] =
              mfma_bf16(*reinterpret_cast<const u32x4*>(&lds.dn[off]), vb_n[kb][ks], dp[qb]);
        }
      }
    };
    u32x4 pa[2][NM], dsa[2][NM];
    // ---- P, dS of block kb, the dV / dK operands and the dS tile
    auto softmax = [&](const int kb, const floatx4 (&s)[QB], const floatx4 (&dp)[QB]) {
      const bool kvalid = !kTail || cb + 16 * kb + li < kh;
      float pv[QBP][4], dsv_[QBP][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        // LSE / Delta of the members this tile gives the lane: 16qb + 4lg + j
        const floatx4 l2 = *reinterpret_cast<const floatx4*>(&lds.lse2[qb * 16 + 4 * lg]);
        const floatx4 dl = *reinterpret_cast<const floatx4*>(&lds.delta[qb * 16 + 4 * lg]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p =
              kvalid ? __builtin_amdgcn_exp2f(fmaf(s[qb][j], c2, -l2[j])) : 0.f;
          pv[qb][j] = p;
          dsv_[qb][j] = p * (dp[qb][j] - dl[j]);
        }
      }
#pragma unroll
      for (int qb = QB; qb < QBP; ++qb)
#pragma unroll
        for (int j = 0; j < 4; ++j) pv[qb][j] = dsv_[qb][j] = 0.f;
      {
        // B operands of dO^T P / Q^T dS: column li <-> key, slot (lg, e) <-> member
        // 16(2m + e/4) + 4lg + e%4
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          pa[kb][m][0] = pack_bf16(pv[2 * m][0], pv[2 * m][1]);
          pa[kb][m][1] = pack_bf16(pv[2 * m][2], pv[2 * m][3]);
          pa[kb][m][2] = pack_bf16(pv[2 * m + 1][0], pv[2 * m + 1][1]);
          pa[kb][m][3] = pack_bf16(pv[2 * m + 1][2], pv[2 * m + 1][3]);
          dsa[kb][m][0] = pack_bf16(dsv_[2 * m][0], dsv_[2 * m][1]);
          dsa[kb][m][1] = pack_bf16(dsv_[2 * m][2], dsv_[2 * m][3]);
          dsa[kb][m][2] = pack_bf16(dsv_[2 * m + 1][0], dsv_[2 * m + 1][1]);
          dsa[kb][m][3] = pack_bf16(dsv_[2 * m + 1][2], dsv_[2 * m + 1][3]);
        }
      }
      // dS tile (unscaled) -> LDS as [key][member]: the lane's 4 members are adjacent
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        *reinterpret_cast<u32x2*>(&lds.ds[(16 * kb + li) * 80 + 16 * qb + 4 * lg]) =
            u32x2{pack_bf16(dsv_[qb][0], dsv_[qb][1]), pack_bf16(dsv_[qb][2], dsv_[qb][3])};
    };
    {
      floatx4 s0[QB], dp0[QB];
      s_dp(0, s0, dp0);
      softmax(0, s0, dp0);
    }
    floatx4 s1[QB], dp1[QB];
    s_dp(1, s1, dp1);
    // ---- K^T operands of dQ^T += K^T dS^T (row li <-> feature 16fb + li, slot (lg, e) <->
    // key 4lg + e for e < 4, 16 + 4lg + e - 4 for e >= 4), made from the natural K rows now:
    // kb_n x sel moves feature block fb of each 16-key tile into the C layout (lane li <->
    // feature, keys 4lg + j), which packed to bf16 is exactly that operand.
    u32x4 kT[NDB];
#pragma unroll
    for (int fb = 0; fb < NDB; ++fb) {
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      const floatx4 t0 = mfma_bf16(kb_n[0][fb >> 1], sel[fb & 1], z);
      const floatx4 t1 = mfma_bf16(kb_n[1][fb >> 1], sel[fb & 1], z);
      kT[fb] = u32x4{pack_bf16(t0[0], t0[1]), pack_bf16(t0[2], t0[3]), pack_bf16(t1[0], t1[1]),
                     pack_bf16(t1[2], t1[3])};
    }
    // The natural K/V registers are free again: request the next chunk's rows (past the end
    // the clamped positions reload the last key) and the keys of the one after, so that the
    // gathers have the rest of this chunk to arrive. The compiler barriers keep them after
    // the MFMAs above and ahead of this chunk's stores.
    asm volatile("" ::: "memory");
    load_nat(nkey);
    load_keys(cb + 64, nkey);
    asm volatile("" ::: "memory");
    softmax(1, s1, dp1);

    // ---- dQ^T += K^T dS^T; the B operand dS^T is read from the LDS tile in the key order
    // of the K^T operands
    wave_lds_fence();   // dS tile complete
    {
      u32x4 bds[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        // transposed reads: lane li gets member 16qb + li of keys 4lg .. 4lg + 3 (lo) and
        // 16 + 4lg .. 16 + 4lg + 3 (hi)
        const int r = 4 * lg + (li >> 2), c = 16 * qb + 4 * (li & 3);
        const u32x2 lo = lds_read_tr16(&lds.ds[r * 80 + c]);
        const u32x2 hi = lds_read_tr16(&lds.ds[(r + 16) * 80 + c]);
        bds[qb] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int fb = 0; fb < NDB; ++fb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) dqacc[qb][fb] = mfma_bf16(kT[fb], bds[qb], dqacc[qb][fb]);
    }

    // ---- dV^T = dO^T P (t = 0), dK^T = Q^T dS (t = 1, dK = scale times it), the 32 x d tiles
    // of both: A operands by transposed LDS reads (row li <-> feature 16fb + li,
    // slot (lg, e) <-> member 32m + 16(e/4) + 4lg + e%4), each read once for both 16-key
    // blocks; lane: key 16kb + li, features 16fb + 4lg + j. Then per block kb its largest
    // |entry| m (the lane's features, the key's 3 other lanes, the block's 16 keys) sets the
    // block's format, the same in every lane:
    //   * true-unit m <= kStage8Bound (d = 128): 8-bit codes 128 + round(x * 127/m); lane
    //     (li, lg) holds bytes 32lg .. 32lg + 31 of row 16kb + li (byte 32lg + 4fb + j <->
    //     feature 16fb + 4lg + j); factor -m/127 (sign bit set, even when m = 0);
    //   * else fp16 times the power of two kStageMax/m rounded down (pow2_scale); feature
    //     blocks in pairs (2fp, 2fp + 1), staging position 32fp + 8lg + t holding feature
    //     32fp + 4lg + t (t < 4) or 32fp + 16 + 4lg + t - 4; factor its reciprocal.
    // Both kinds of row start the row's 2d-byte place. Lanes li and li ^ 8 swap 16-byte
    // granules (DPP row_ror:8 with a bank mask: lanes 8..15 of each row take the other half
    // of lane li - 8, lanes 0..7 of lane li + 8), so every store writes 8 whole 128-byte
    // lines. The rows are written once and read back by the reduce long after, so the stores
    // are non-temporal; they are the bulk of this kernel's HBM traffic.
    float fac[2][2];   // [t][kb]: what the reduce multiplies the staged entries by
    const long long r0 = grow + cb + (li & 7);
    auto swap_store = [&](const u32x4& lo, const u32x4& hi, uint16_t* dst, long long ra,
                          int col16) {
      u32x4 s1, s2;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        s1[w] = __builtin_amdgcn_update_dpp(lo[w], hi[w], 0x128, 0xf, 0xc, false);
        s2[w] = __builtin_amdgcn_update_dpp(hi[w], lo[w], 0x128, 0xf, 0x3, false);
      }
      __builtin_nontemporal_store(s1, reinterpret_cast<u32x4*>(dst + ra * D + col16));
      __builtin_nontemporal_store(s2, reinterpret_cast<u32x4*>(dst + (ra + 8) * D + col16));
    };
    // both tensors' tiles first (their MFMAs overlap the other tile's encoding)
    floatx4 acc2[2][NDB][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int fb = 0; fb < NDB; ++fb) acc2[t][fb][0] = acc2[t][fb][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int fb = 0; fb < NDB; ++fb)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int r1 = 32 * m + 4 * lg + (li >> 2);
        const int c = 16 * fb + 4 * (li & 3);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint16_t* a = t == 0 ? lds.dn : lds.qn;
          const u32x2 a1 = lds_read_tr16(&a[swz<D>(r1, c)]);
          const u32x2 a2 = lds_read_tr16(&a[swz<D>(r1 + 16, c)]);
          const u32x4 aT = {a1[0], a1[1], a2[0], a2[1]};
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            acc2[t][fb][kb] = mfma_bf16(aT, t == 0 ? pa[kb][m] : dsa[kb][m], acc2[t][fb][kb]);
        }
      }
    // the four blocks' largest |entries| (tile units), then their formats
    float mx4[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float mx = 0.f;
#pragma unroll
        for (int fb = 0; fb < NDB; ++fb)
#pragma unroll
          for (int j = 0; j < 4; ++j) mx = fmaxf(mx, fabsf(acc2[t][fb][kb][j]));
        mx4[t][kb] = max_in_row16(max_over_rows(mx));
      }
    auto is8 = [&](int t, int kb) {
      return kStage8<D> && mx4[t][kb] * (t == 0 ? 1.f : scale) <= kStage8Bound;
    };
    auto enc8 = [&](int t, int kb) {
      const float mx = mx4[t][kb];
      // |x| <= m and 127 * rcp(m) exceeds 127/m by at most an ulp: |x * inv| < 127.5
      const float inv = mx > 0.f ? 127.f * __builtin_amdgcn_rcpf(mx) : 0.f;
      fac[t][kb] = -(mx * (1.f / 127.f)) * (t == 0 ? 1.f : scale);
      u32x4 g0, g1;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        g0[w] = pack_i8(acc2[t][w][kb], inv);
        g1[w] = pack_i8(acc2[t][(w + 4) % NDB][kb], inv);
      }
      swap_store(g0, g1, t == 0 ? cv : ck, r0 + 16 * kb, 16 * lg + 8 * (li >> 3));
    };
    auto enc16 = [&](int t, int kb) {
      const float sc = pow2_scale(mx4[t][kb]);   // a power of two: its reciprocal is exact
      fac[t][kb] = sc > 0.f ? __builtin_amdgcn_rcpf(sc) * (t == 0 ? 1.f : scale) : 0.f;
#pragma unroll
      for (int fp = 0; fp < NDB / 2; fp += 2) {
        u32x4 x[2];   // granules of feature-block pairs fp (even) and fp + 1 (odd)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const floatx4& e0 = acc2[t][2 * (fp + h2)][kb];
          const floatx4& e1 = acc2[t][2 * (fp + h2) + 1][kb];
          x[h2] = u32x4{pack_f16(e0[0] * sc, e0[1] * sc), pack_f16(e0[2] * sc, e0[3] * sc),
                        pack_f16(e1[0] * sc, e1[1] * sc), pack_f16(e1[2] * sc, e1[3] * sc)};
        }
        // lane: granules 8p + lg (even pair) and 8p + 4 + lg (odd) of row li, p = fp/2
        swap_store(x[0], x[1], t == 0 ? cv : ck, r0 + 16 * kb,
                   8 * (8 * (fp >> 1) + 4 * (li >> 3) + lg));
      }
    };
    // all four blocks 8-bit (nearly every chunk on the workloads here): one straight run;
    // otherwise block by block (each branch the same in every lane)
    if (__builtin_amdgcn_readfirstlane((int)(is8(0, 0) && is8(0, 1) && is8(1, 0) && is8(1, 1)))) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) enc8(t, kb);
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (__builtin_amdgcn_readfirstlane((int)is8(t, kb)))
            enc8(t, kb);
          else
            enc16(t, kb);
        }
    }
    // both blocks' factors in one 16-byte store by every lane (one address, unconditional);
    // (grow + cb) is a multiple of 32, so the pair is 16-byte aligned
    *reinterpret_cast<float4*>(&bfac[(grow + cb) / 16]) =
        make_float4(fac[0][0], fac[1][0], fac[0][1], fac[1][1]);
    wave_lds_fence();   // the next chunk overwrites the dS tile
  };
  // full chunks carry no key masks; the partial last chunk is its own instantiation
  const int kfull = kh & ~31;
  if (kfull == 0) {
    chunk(0, Flag<true>{});
  } else {
    chunk(0, Flag<false>{});
    for (int cb = 32; cb < kfull; cb += 32) chunk(cb, Flag<false>{});
    if (kfull < kh) chunk(kfull, Flag<true>{});
  }

  // ---- store dQ (fp32): lane holds member 16qb + li, features 16fb + 4lg + j
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int n = gg.token(g, qb * 16 + li);
    float* drow = dq + base + (long long)n * D;
#pragma unroll
    for (int fb = 0; fb < NDB; ++fb)
      *reinterpret_cast<float4*>(drow + 16 * fb + 4 * lg) =
          make_float4(dqacc[qb][fb][0] * scale, dqacc[qb][fb][1] * scale,
                      dqacc[qb][fb][2] * scale, dqacc[qb][fb][3] * scale);
  }
}

// fp32 inputs: lane = group member for P/dS/dQ, then lane = feature for dK/dV.
// fp32 dK/dV: each group's partial sum is rounded to a multiple of 2^-32 and added as a 64-bit
// integer. Integer sums do not depend on the order of the atomics, so dK/dV repeat bit for bit
// whatever the scheduling; each contribution is off by at most 2^-33 (sums must stay below
// 2^31 in magnitude).
__device__ __forceinline__ unsigned long long to_fixed(float x) {
  return (unsigned long long)__double2ll_rn((double)x * 4294967296.0);
}
__global__ void fixed_to_f32(const unsigned long long* __restrict__ acc, float* __restrict__ out,
                             long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = (float)((double)(long long)acc[i] * (1.0 / 4294967296.0));
}

// fp32 inputs: v_mfma_f32_16x16x4_f32 tiles, one wave per group, keys in chunks of 16. The
// group's Q and dO rows and each chunk's K and V rows sit in LDS (rows padded by one word);
// S^T = K Q^T and dP^T = V dO^T give a lane 4 keys of one query, P and dS go to LDS tiles
// [key][query], and dQ^T += K^T dS^T, dV^T = dO^T P, dK^T = Q^T dS (the last two over the
// group's queries) come out of more tiles. Each chunk's dV/dK rows are added to the
// fixed-point accumulators; dQ is written once. Kept simple (it serves fp32 inputs).
template <int D, int QB>
__global__ __launch_bounds__(64) void attn_bwd_f32(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ o, const float* __restrict__ d_o, const float* __restrict__ lse,
    const int32_t* __restrict__ idx, float scale, float* __restrict__ dq,
    unsigned long long* __restrict__ acck, unsigned long long* __restrict__ accv, Geom geo) {
  constexpr int G = 16 * QB;
  constexpr int DP = D + 1;   // LDS row stride of Q, dO, K, V (words)
  constexpr int GP = G + 1;   // LDS row stride of the P and dS tiles
  constexpr int NDB = D / 16;
  extern __shared__ float smem[];
  float* const sq = smem;            // [G][DP]
  float* const sdo = sq + G * DP;    // [G][DP]
  float* const sk = sdo + G * DP;    // [16][DP]
  float* const sv = sk + 16 * DP;    // [16][DP]
  float* const sp = sv + 16 * DP;    // [16][GP]: P[key][query]
  float* const sds = sp + 16 * GP;   // [16][GP]: dS[key][query]
  const int lane = threadIdx.x;
  const int lg = lane >> 4;
  const int li = lane & 15;
  int b, h, g;
  decode_unit(geo, blockIdx.x, b, h, g);
  const int kh = geo.k[h];
  const long long bh = (long long)b * geo.H + h;
  const long long base = bh * geo.S * D;
  const int32_t* row = idx + geo.row_offset(b, h, g);
  const GroupGeom gg{geo.Hh, geo.W, geo.gt, geo.gh, geo.gw, geo.nbh, geo.nbw};
  for (int i = lane; i < G * D; i += 64) {
    const int r = i / D, c = i - r * D;
    const long long n = gg.token(g, r);
    sq[r * DP + c] = q[base + n * D + c];
    sdo[r * DP + c] = d_o[base + n * D + c];
  }
  __syncthreads();
  // LSE and Delta = dO . O of the lane's query 16qb + li (features lg, lg + 4, .. summed over
  // the 4 lanes of the query)
  float lq[QB], dl[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const long long n = gg.token(g, 16 * qb + li);
    lq[qb] = lse[bh * geo.S + n];
    float acc = 0.f;
    for (int c = lg; c < D; c += 4) acc = fmaf(sdo[(16 * qb + li) * DP + c], o[base + n * D + c], acc);
    acc += __shfl_xor(acc, 16, 64);
    acc += __shfl_xor(acc, 32, 64);
    dl[qb] = acc;
  }
  floatx4 dqacc[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int f = 0; f < NDB; ++f) dqacc[qb][f] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int cb = 0; cb < kh; cb += 16) {
    // lane li's key (positions past the row end read its last key; their P and dS are 0)
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
      // S^T and dP^T: lane holds keys 4lg + j of the chunk for query 16qb + li
      floatx4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int st = 0; st < D / 4; ++st) {
        s = mfma_f32(sk[li * DP + 4 * st + lg], sq[(16 * qb + li) * DP + 4 * st + lg], s);
        dp = mfma_f32(sv[li * DP + 4 * st + lg], sdo[(16 * qb + li) * DP + 4 * st + lg], dp);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = cb + 4 * lg + j < kh;
        const float p = ok ? expf(fmaf(s[j], scale, -lq[qb])) : 0.f;
        sp[(4 * lg + j) * GP + 16 * qb + li] = p;
        sds[(4 * lg + j) * GP + 16 * qb + li] = p * (dp[j] - dl[qb]);
      }
    }
    // (the P and dS tiles are this wave's own LDS writes, read back in order)
    // dQ^T += K^T dS^T: lane holds features 16f + 4lg + j of query 16qb + li
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int f = 0; f < NDB; ++f)
#pragma unroll
        for (int st = 0; st < 4; ++st)
          dqacc[qb][f] = mfma_f32(sk[(4 * st + lg) * DP + 16 * f + li],
                                  sds[(4 * st + lg) * GP + 16 * qb + li], dqacc[qb][f]);
    // dV^T = dO^T P and dK^T = Q^T dS over the group's queries: lane holds features
    // 16f + 4lg + j of chunk key li
    const bool kvalid = cb + li < kh;
    const long long kr = base + (long long)key * D;
#pragma unroll 1
    for (int f = 0; f < NDB; ++f) {
      floatx4 tv = {0.f, 0.f, 0.f, 0.f}, tk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < G / 4; ++st) {
        tv = mfma_f32(sdo[(4 * st + lg) * DP + 16 * f + li], sp[li * GP + 4 * st + lg], tv);
        tk = mfma_f32(sq[(4 * st + lg) * DP + 16 * f + li], sds[li * GP + 4 * st + lg], tk);
      }
      if (kvalid) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          atomicAdd(accv + kr + 16 * f + 4 * lg + j, to_fixed(tv[j]));
          atomicAdd(acck + kr + 16 * f + 4 * lg + j, to_fixed(tk[j] * scale));
        }
      }
    }
    __syncthreads();   // the next chunk's rows overwrite the tiles
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const long long n = gg.token(g, 16 * qb + li);
#pragma unroll
    for (int f = 0; f < NDB; ++f)
      *reinterpret_cast<floatx4*>(dq + base + n * D + 16 * f + 4 * lg) = dqacc[qb][f] * scale;
  }
}

}  // namespace

// Workspace layout for a chunk capacity of `cs` slots and `e` staging rows:
//   [rs: cs*NG*(nB+1) u32][rsT: cs*NG*(nB+1) u32][tot: cs*(nB+1) u32][off: cs*(nB+1) u32]
//   [perm: e u32][block factors: e/16 float2][dV rows: e*d fp16][dK rows: e*d fp16], every
//   region 256-byte aligned (an 8-bit row uses the first d bytes of its fp16 row's place).
struct WsLayout {
  size_t rs, rst, tot, off, perm, fac, cv, ck, total;
};
static WsLayout ws_layout(const Geom& geo, long long cs, long long e) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nb = (size_t)n_buckets(geo.S);
  WsLayout L;
  L.rs = 0;
  L.rst = L.rs + al(cs * geo.NG * (nb + 1) * 4);
  L.tot = L.rst + al(cs * geo.NG * (nb + 1) * 4);
  L.off = L.tot + al(cs * (nb + 1) * 4);
  L.perm = L.off + al(cs * (nb + 1) * 4);
  L.fac = L.perm + al((size_t)e * 4);
  L.cv = L.fac + al((size_t)e / 16 * 8);
  L.ck = L.cv + al((size_t)e * geo.d * sizeof(uint16_t));
  L.total = L.ck + (size_t)e * geo.d * sizeof(uint16_t);
  return L;
}

static long long max_slot_rows(const Geom& geo) {
  int kmax = 0;
  for (int h = 0; h < geo.H; ++h) kmax = std::max(kmax, geo.k[h]);
  return (long long)geo.NG * padded_k(kmax);
}

size_t bwd_workspace_bytes(const Geom& geo) {
  // fp32 path: the dV and dK fixed-point accumulators, 8 bytes per element each
  if (geo.dtype == DSV_FP32) return (size_t)geo.B * geo.H * geo.S * geo.d * 2 * sizeof(uint64_t);
  return ws_layout(geo, 1, max_slot_rows(geo)).total;
}

// Chunk capacity for a workspace: cs slots, ecap staging rows.
static void chunk_capacity(const Geom& geo, size_t ws_bytes, long long& cs, long long& ecap) {
  const int nslots = geo.B * geo.H;
  const long long e1 = max_slot_rows(geo);
  cs = std::min<long long>(kMaxChunk, nslots);
  while (cs > 1 && ws_layout(geo, cs, e1).total > ws_bytes) --cs;
  ecap = e1;   // largest row capacity for this slot capacity
  const size_t per_row = 4 + 1 + 2 * (size_t)geo.d * sizeof(uint16_t);
  const size_t fixed = ws_layout(geo, cs, 0).total;
  if (ws_bytes > fixed) ecap = std::max<long long>(e1, (long long)((ws_bytes - fixed) / per_row) - 64);
  while (ecap > e1 && ws_layout(geo, cs, ecap).total > ws_bytes) ecap -= 64;
}

// Next chunk of consecutive slots from s0 (at most cs slots, at most ecap staging rows).
static Chunk next_chunk(const Geom& geo, int s0, long long cs, long long ecap) {
  const int nslots = geo.B * geo.H;
  Chunk ch;
  ch.s0 = s0;
  ch.n = 0;
  long long rows = 0;
  while (s0 + ch.n < nslots && ch.n < cs) {
    const int h = geo.order[(s0 + ch.n) / geo.B];
    const long long r = (long long)geo.NG * padded_k(geo.k[h]);
    if (ch.n > 0 && rows + r > ecap) break;
    ch.edge_base[ch.n] = rows;
    rows += r;
    ++ch.n;
  }
  ch.edge_base[ch.n] = rows;
  return ch;
}

int bwd_chunk_count(const Geom& geo, size_t ws_bytes) {
  if (geo.dtype == DSV_FP32) return 1;
  long long cs, ecap;
  chunk_capacity(geo, ws_bytes, cs, ecap);
  int n = 0;
  for (int s0 = 0; s0 < geo.B * geo.H; ++n) s0 += next_chunk(geo, s0, cs, ecap).n;
  return n;
}

// ---- the no-allocation backward's scratch: one fixed device array per GPU, in place of a
// caller workspace. In host code `scratch` is only a stand-in for the symbol: its device
// address is looked up once per device (hipGetSymbolAddress, with that device current) and
// only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[DSV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

int bwd_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

int launch_attn_bwd(const Geom& geo, const void* q, const void* k, const void* v, const void* o,
                    const void* d_o, const float* lse, const int32_t* idx, float scale, float* dq,
                    float* dk, float* dv, void* ws, size_t ws_bytes, void* stream,
                    void* const* events) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  // optional profiling marks: events[4c + i] before the chunk's pre-passes (i = 0), its
  // backward kernel (1) and its reduce (2), and after the reduce (3)
  auto mark = [&](int i) {
    if (events) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), st);
  };
  if (geo.dtype == DSV_FP32) {
    // fixed-point accumulators in the workspace (dK, then dV), zeroed, then converted
    const long long n = (long long)geo.B * geo.H * geo.S * geo.d;
    unsigned long long* acck = static_cast<unsigned long long*>(ws);
    unsigned long long* accv = acck + n;
    const long long n4 = n * 2 * (long long)sizeof(uint64_t) / 16;   // float4 units of both
    const int fill_blocks = (int)std::min<long long>((n4 + 255) / 256, 4096);
    hipLaunchKernelGGL(fill_zero, dim3(fill_blocks), dim3(256), 0, st, (float4*)ws, n4);
    const int conv_blocks = (int)std::min<long long>((n + 255) / 256, 4096);
    const dim3 grid(geo.B * geo.H * geo.NG);
    const int QB32 = geo.G / 16;
    // LDS: Q and dO rows, the chunk's K and V rows (rows padded by one word), P and dS tiles
    const size_t shm =
        ((size_t)2 * (geo.G + 16) * (geo.d + 1) + (size_t)2 * 16 * (geo.G + 1)) * sizeof(float);
#define DSV_BWD32(DD, QQ)                                                                     \
  if (geo.d == DD && QB32 == QQ) {                                                            \
    if (shm > 65536)                                                                          \
      (void)hipFuncSetAttribute((const void*)attn_bwd_f32<DD, QQ>,                            \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);        \
    hipLaunchKernelGGL((attn_bwd_f32<DD, QQ>), grid, dim3(64), shm, st, (const float*)q,      \
                       (const float*)k, (const float*)v, (const float*)o, (const float*)d_o,  \
                       lse, idx, scale, dq, acck, accv, geo);                                 \
    hipLaunchKernelGGL(fixed_to_f32, dim3(conv_blocks), dim3(256), 0, st, acck, dk, n);      \
    hipLaunchKernelGGL(fixed_to_f32, dim3(conv_blocks), dim3(256), 0, st, accv, dv, n);      \
    return (int)hipGetLastError();                                                            \
  }
    DSV_BWD32(64, 1) DSV_BWD32(64, 2) DSV_BWD32(64, 3) DSV_BWD32(64, 4)
    DSV_BWD32(128, 1) DSV_BWD32(128, 2) DSV_BWD32(128, 3) DSV_BWD32(128, 4)
#undef DSV_BWD32
    return (int)hipErrorInvalidValue;
  }

  // ---- bf16 path: chunks of (b, h) slots sized to the workspace
  const int nslots = geo.B * geo.H;
  long long cs, ecap;
  chunk_capacity(geo, ws_bytes, cs, ecap);
  const WsLayout L = ws_layout(geo, cs, ecap);
  char* wsb = static_cast<char*>(ws);
  uint32_t* rs = reinterpret_cast<uint32_t*>(wsb + L.rs);
  uint32_t* rsT = reinterpret_cast<uint32_t*>(wsb + L.rst);
  uint32_t* tot = reinterpret_cast<uint32_t*>(wsb + L.tot);
  uint32_t* off = reinterpret_cast<uint32_t*>(wsb + L.off);
  uint32_t* perm = reinterpret_cast<uint32_t*>(wsb + L.perm);
  float2* bfac = reinterpret_cast<float2*>(wsb + L.fac);
  uint16_t* cv = reinterpret_cast<uint16_t*>(wsb + L.cv);
  uint16_t* ck = reinterpret_cast<uint16_t*>(wsb + L.ck);
  const int nB = n_buckets(geo.S);
  const int QBn = geo.G / 16;

  int s0 = 0;
  for (int c = 0; s0 < nslots; ++c) {
    const Chunk ch = next_chunk(geo, s0, cs, ecap);
    const int rows_waves = ch.n * geo.NG;
    mark(4 * c);
    hipLaunchKernelGGL(row_bucket_starts, dim3((rows_waves + 3) / 4), dim3(256), 0, st, idx, ch,
                       rs, geo);
    const int ttiles = ch.n * ((nB + 64) / 64) * ((geo.NG + 63) / 64);
    hipLaunchKernelGGL(transpose_rs, dim3(ttiles), dim3(256), 0, st, rs, rsT, geo);
    hipLaunchKernelGGL(bucket_totals, dim3(ch.n * nB), dim3(64), 0, st, rsT, tot, geo);
    hipLaunchKernelGGL(bucket_offsets, dim3(ch.n), dim3(256), 0, st, tot, off, geo);
    // the first sweep's masks stay in LDS up to 6144 groups (48 KB)
    const int cached = geo.NG <= 6144 ? 1 : 0;
    hipLaunchKernelGGL(bucket_perm, dim3(ch.n * nB), dim3(64 * kPermWaves),
                       cached ? geo.NG * sizeof(uint2) : 0,
                       st, rsT, off, idx, ch, perm, geo, cached);
    mark(4 * c + 1);
#define DSV_BWD16(DD, QQ)                                                                       \
  if (geo.d == DD && QBn == QQ) {                                                               \
    hipLaunchKernelGGL((attn_bwd_bf16<DD, QQ>), dim3(rows_waves), dim3(64), 0, st,              \
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,              \
                       (const uint16_t*)o, (const uint16_t*)d_o, lse, idx, scale, dq, ch, cv,   \
                       ck, bfac, geo);                                                          \
    mark(4 * c + 2);                                                                            \
    hipLaunchKernelGGL((bucket_reduce<DD>), dim3(ch.n * nB * 2), dim3(64), 0, st, off, perm,    \
                       bfac, cv, ck, ch, dk, dv, geo);                                          \
    mark(4 * c + 3);                                                                            \
  } else
    DSV_BWD16(64, 1) DSV_BWD16(64, 2) DSV_BWD16(64, 3) DSV_BWD16(64, 4)
    DSV_BWD16(128, 1) DSV_BWD16(128, 2) DSV_BWD16(128, 3) DSV_BWD16(128, 4)
    return (int)hipErrorInvalidValue;
#undef DSV_BWD16
    const int e = (int)hipGetLastError();
    if (e) return e;
    s0 += ch.n;
  }
  return 0;
}

}  // namespace dsv
