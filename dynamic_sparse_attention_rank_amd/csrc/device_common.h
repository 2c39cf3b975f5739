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

// 32 x 32 tiles: A (32 x 16) lane l holds row l % 32, 8 contraction elements of slot l / 32;
// B likewise for column l % 32; C element 4i + j of lane l is row 8i + 4(l / 32) + j, column
// l % 32. The fp32 form contracts one element per slot.
typedef float floatx16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ floatx16 mfma32_bf16(const u32x4& a, const u32x4& b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mfma32_f32(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
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

// Sum over the four 16-lane rows: lane l gets v(l%16) + v(l%16 + 16) + v(l%16 + 32) +
// v(l%16 + 48), paired as (r0 + r1) + (r2 + r3), the same in every lane. gfx950's row swaps
// (v_permlane16_swap / v_permlane32_swap) move the data without an LDS round trip: with both
// operands v, the two results of a swap hold the two rows of each pair.
__device__ __forceinline__ float sum_over_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Maximum over the four 16-lane rows: lane l gets max of v(l%16 + 16r), r < 4, by the same
// row swaps as sum_over_rows.
__device__ __forceinline__ float max_over_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Four values to biased 8-bit codes in one word (byte j <- x[j]): code = 128 + round-to-
// nearest-even(x[j] * inv), for |x[j] * inv| < 127.5. Adding 1.5 * 2^23 + 128 in one fused
// multiply-add leaves exactly that integer in the low mantissa bits (the sum lies in
// [2^23, 2^24), where the float spacing is 1), so the code is the low byte of the result.
__device__ __forceinline__ uint32_t pack_i8(const floatx4& x, float inv) {
  constexpr float kMagic = 12583040.f;   // 0x4b400080
  const uint32_t y0 = __float_as_uint(fmaf(x[0], inv, kMagic));
  const uint32_t y1 = __float_as_uint(fmaf(x[1], inv, kMagic));
  const uint32_t y2 = __float_as_uint(fmaf(x[2], inv, kMagic));
  const uint32_t y3 = __float_as_uint(fmaf(x[3], inv, kMagic));
  const uint32_t p01 = __builtin_amdgcn_perm(y1, y0, 0x0c0c0400u);   // bytes: y0.b0, y1.b0
  const uint32_t p23 = __builtin_amdgcn_perm(y3, y2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}

// Maximum over each 16-lane row (every lane of the row gets it), by DPP: swaps inside quads,
// then rotations by 4 and 8 lanes.
__device__ __forceinline__ float max_in_row16(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf,
                                                          false)));   // quad_perm 1,0,3,2
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf,
                                                          false)));   // quad_perm 2,3,0,1
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf,
                                                          false)));   // row_ror 4
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf,
                                                          false)));   // row_ror 8
  return v;
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// Key indices come from caller memory: clamp them into [0, S) so that a bad list can never
// address outside K/V (the result for such a list is unspecified, but memory-safe).
// Compile-time switch passed to generic lambdas (e.g. the last, partial key chunk).
template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// A key from an index list, clamped into [0, S) as an unsigned value: a negative key reads key
// S - 1, like one >= S (one instruction; only malformed lists hold such keys).
__device__ __forceinline__ int clamp_key(int key, int S) {
  return (int)min((uint32_t)key, (uint32_t)S - 1u);
}

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


// ---- LDS row copies read both ways -----------------------------------------------------------
// A [row][feature] bf16 tile with D features per row, chunk c (8 features, 16 bytes) of row r
// stored at chunk position c ^ (r mod D/8): 16-byte reads of one chunk from 16 consecutive
// rows hit distinct banks, and the 8-byte transposed reads below stay inside one chunk.
// element offset of feature `col` (col % 4 == 0) of row r in the swizzled layout
template <int D>
__device__ __forceinline__ int swz(int r, int col) {
  return r * D + ((((col >> 3) ^ r) & (D / 8 - 1)) << 3) + (col & 7);
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane l's bytes
// land at lds_base + 16 l. lds_base must be the same in every lane. The transfer is counted by
// vmcnt like any vector load; the data may be read from LDS once that count has drained.
__device__ __forceinline__ void global_load_lds16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_base, 16, 0,
                                   0);
}
// Wait until at most N vector memory operations of this wave are outstanding, and keep memory
// accesses on their side. Rows brought in by direct-to-LDS loads are read only after N = 0:
// their retirement order relative to ordinary loads is not relied on.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ds_read_b64_tr_b16: within each 16-lane block, lane j passes the address of 4 elements
// (row R0 + j/4, columns C0 + 4(j%4)) and lane i receives column C0 + i of rows R0 .. R0 + 3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)((__attribute__((address_space(3))) const uint16_t*)p));
  return __builtin_bit_cast(u32x2, v);
}


// 0/1 selection operands: sel[h] as the B operand of a 16x16x32 MFMA maps contraction slot
// (lg, e) <-> feature 32ks + 8lg + e to output column li iff 8lg + e == 16h + li, so
// A x sel[h] copies features 32ks + 16h .. + 15 of the A rows into the C layout: lane li then
// holds feature 32ks + 16h + li of A rows 4lg + j. Exact for bf16 A (one product by 1.0).
__device__ __forceinline__ void make_selection(int lane, u32x4 sel[2]) {
  const int lg = lane >> 4, li = lane & 15;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = (8 * lg + 2 * w == 16 * hh + li) ? 0x3f80u : 0u;
      const uint32_t hi = (8 * lg + 2 * w + 1 == 16 * hh + li) ? 0x3f80u : 0u;
      sel[hh][w] = lo | (hi << 16);
    }
}

}  // namespace dsv
