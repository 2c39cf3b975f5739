// device_common.h — gfx950 (CDNA4) building blocks shared by the DSV kernels.
//
// MFMA operand conventions used throughout (wave64; lane = 16*lg + li, lg in 0..3, li in 0..15):
//   v_mfma_f32_16x16x32_bf16:  A (16 x 32): lane holds row li, 8 contraction elements of slot lg.
//                              B (32 x 16): lane holds column li, 8 contraction elements of slot lg.
//                              C (16 x 16): lane holds column li, rows 4*lg + j (j = 0..3).
//   v_mfma_f32_16x16x4_f32:    A, B: one contraction element per lane (slot lg); C as above.
// Only the row/column placement matters for correctness: the contraction elements may be
// assigned to (lg, e) slots in any order, as long as A and B use the same assignment, so the
// kernels permute keys and feature dimensions freely inside a contraction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx4 mfma_bf16(const u32x4& a, const u32x4& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma_f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Two floats -> packed bf16 pair (round to nearest even), `lo` in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ float bf16_round(float x) {  // value of the nearest bf16
  return bf16_lo(pack_bf16(x, 0.0f));
}

// Low 16-bit halves of a (-> bits 0..15) and b (-> bits 16..31).
__device__ __forceinline__ uint32_t pack_lo_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
// High 16-bit halves of a (-> bits 0..15) and b (-> bits 16..31).
__device__ __forceinline__ uint32_t pack_hi_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// 8 x 8 transpose of 16-bit elements held by one lane: in[e] holds 8 consecutive features of
// item e (two per dword); out[f] holds feature f of items 0..7 (two per dword).
__device__ __forceinline__ void transpose8x8_b16(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int f2 = 0; f2 < 4; ++f2) {      // features 2*f2 (lo halves) and 2*f2+1 (hi halves)
#pragma unroll
    for (int u = 0; u < 4; ++u) {       // items 2u, 2u+1
      out[2 * f2][u] = pack_lo_halves(in[2 * u][f2], in[2 * u + 1][f2]);
      out[2 * f2 + 1][u] = pack_hi_halves(in[2 * u][f2], in[2 * u + 1][f2]);
    }
  }
}

// Same for 8 items x 4 features (each item holds 4 features in two dwords): out[f] holds
// feature f of items 0..7.
__device__ __forceinline__ void transpose8x4_b16(const u32x2 in[8], u32x4 out[4]) {
#pragma unroll
  for (int f2 = 0; f2 < 2; ++f2) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      out[2 * f2][u] = pack_lo_halves(in[2 * u][f2], in[2 * u + 1][f2]);
      out[2 * f2 + 1][u] = pack_hi_halves(in[2 * u][f2], in[2 * u + 1][f2]);
    }
  }
}

__device__ __forceinline__ float wave_xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
// Ordering point for the LDS accesses of a single-wave workgroup: waits for this wave's
// outstanding LDS operations and keeps the compiler from moving memory accesses across it.
// __syncthreads() would also wait for every outstanding global load and store (its fence),
// which serialises streaming stores and prefetches with the computation.
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ float wave_xor_sum(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// Key indices come from caller memory: clamp them into [0, S) so that a bad list can never
// address outside K/V (the result for such a list is unspecified, but memory-safe).
__device__ __forceinline__ int clamp_key(int key, int S) { return min(max(key, 0), S - 1); }

// Token index of member j of group g (groups are gt x gh x gw boxes of the T x Hh x W grid,
// numbered row-major; members row-major over (dt, dy, dx)).
struct GroupGeom {
  int Hh, W, gt, gh, gw, nbh, nbw;  // nbh = Hh/gh, nbw = W/gw
  __device__ __forceinline__ int token(int g, int j) const {
    const int a = g / (nbh * nbw);
    const int rem = g - a * (nbh * nbw);
    const int b = rem / nbw;
    const int c = rem - b * nbw;
    const int ghw = gh * gw;
    const int dt = j / ghw;
    const int r2 = j - dt * ghw;
    const int dy = r2 / gw;
    const int dx = r2 - dy * gw;
    return ((a * gt + dt) * Hh + (b * gh + dy)) * W + (c * gw + dx);
  }
};

}  // namespace dsv
