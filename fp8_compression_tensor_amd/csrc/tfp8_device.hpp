// tfp8_device.hpp - wavefront primitives for the gfx950 FP8 ASH + DS kernels.
//
// Everything here works on one 64-lane wavefront.  A "group" is the set of L consecutive
// lanes (L = 4, 8, 16 or 32) that hold one block; group reductions and butterflies only use
// lane exchanges that stay inside the group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tfp8 {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// DPP lane-select controls (gfx9 encoding).
enum : int {
  kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]: lane i reads lane i^1
  kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]: lane i reads lane i^2
  kDppHalfMirror = 0x141, // lane i reads lane i^7 inside each group of 8
  kDppRowMirror = 0x140,  // lane i reads lane i^15 inside each row of 16
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// lane i reads lane i^16 (ds_swizzle bit mode inside 32-lane halves: and 0x1F, xor 0x10)
__device__ __forceinline__ float swz_xor16(float v) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// Integer max over the L lanes of a group; every lane of the group gets the result.  After the
// xor-1 and xor-2 steps all lanes of a quad agree, so the mirror steps (xor 7, xor 15) combine
// whole quads / half-rows exactly like xor 4 / xor 8 would.
template <int L>
__device__ __forceinline__ int group_max_i(int v) {
  static_assert(L == 4 || L == 8 || L == 16 || L == 32, "group of 4, 8, 16 or 32 lanes");
  v = max(v, dpp_i<kDppXor1>(v));
  v = max(v, dpp_i<kDppXor2>(v));
  if constexpr (L >= 8) v = max(v, dpp_i<kDppHalfMirror>(v));
  if constexpr (L >= 16) v = max(v, dpp_i<kDppRowMirror>(v));
  if constexpr (L >= 32) v = max(v, __builtin_amdgcn_ds_swizzle(v, 0x401F));
  return v;
}

// Max over the L lanes of a group of magnitudes (values >= +0); every lane of the group gets
// the result.  Non-negative floats order like their bit patterns read as signed integers, so
// the max runs on the integers: an integer max needs no NaN canonicalisation, which lets the
// compiler fold each lane exchange into the max itself (one v_max_i32 with a DPP operand per
// step instead of a move and two float maxes).
template <int L>
__device__ __forceinline__ float group_max(float v) {
  return __int_as_float(group_max_i<L>(__float_as_int(v)));
}

template <int L>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(L == 4 || L == 8 || L == 16 || L == 32, "group of 4, 8, 16 or 32 lanes");
  v = v + dpp<kDppXor1>(v);
  v = v + dpp<kDppXor2>(v);
  if constexpr (L >= 8) v = v + dpp<kDppHalfMirror>(v);
  if constexpr (L >= 16) v = v + dpp<kDppRowMirror>(v);
  if constexpr (L >= 32) v = v + swz_xor16(v);
  return v;
}

// Sum of the squares of the N values a lane holds of one block.  From N = 32 on (B >= 256) the
// sum runs in float64, where every square of a float32 value is exact and the additions lose
// nothing that matters, and is rounded to float32 once: a float32 sum of 64 similar squares
// (B = 512), even in 8 partial sums, left alpha within a few percent of the 1e-6 bar, and over
// it once with the other roundings of the exact accumulation path.  Shorter sums stay in float32
// (sequential: 16 terms at most, and fewer registers).  With SCALED, the squares are those of
// v[r] * c (each product rounded to float32 first).
template <int N, bool SCALED = false>
__device__ __forceinline__ float sum_squares(const float *v, float c = 1.0f) {
  if constexpr (N < 32) {
    float acc = 0.0f;
#pragma unroll
    for (int r = 0; r < N; ++r) {
      const float u = SCALED ? v[r] * c : v[r];
      acc = fmaf(u, u, acc);
    }
    return acc;
  } else {
    double acc = 0.0;
#pragma unroll
    for (int r = 0; r < N; ++r) {
      const double u = (double)(SCALED ? v[r] * c : v[r]);
      acc = fma(u, u, acc);
    }
    return (float)acc;
  }
}

// Unnormalised Walsh-Hadamard transform of the N values a lane holds (natural order), over
// register strides H0 <= h < HN: H0 = 2 when the stride-1 stage was done at load time, and
// HN < N transforms each run of HN registers on its own.
template <int N, int H0 = 1, int HN = N>
__device__ __forceinline__ void fwht_registers(float (&v)[N]) {
#pragma unroll
  for (int h = H0; h < HN; h <<= 1) {
#pragma unroll
    for (int i = 0; i < N; i += 2 * h) {
#pragma unroll
      for (int k = i; k < i + h; ++k) {
        const float a = v[k], b = v[k + h];
        v[k] = a + b;
        v[k + h] = a - b;
      }
    }
  }
}

// Hadamard transform across the 8 lanes of a group, one instruction per value and stage:
// v_fmac_f32 with a DPP-selected partner, value <- value + sigma * partner, where sigma = -1 on
// the lane of each pair that keeps the difference.  Partners are lane^7 first (DPP has no
// xor-4 lane select), then lane^1 and lane^2, with sigma from lane bits 2, 0 and 1.  Mask 7 =
// 4 ^ 3, so the three masks still span all lane bits; the network computes a signed
// permutation of the natural transform: lane j ends with lane8_sign(j) * (H_8 v)[lane8_perm(j)]
// (worked out by enumerating the network on the unit vectors).
__device__ __forceinline__ int lane8_perm(int j) {
  // 0,5,6,3,4,1,2,7: bit 2 flips when bits 0 and 1 differ
  return j ^ (((j ^ (j >> 1)) & 1) << 2);
}
__device__ __forceinline__ float lane8_sign(int j) {
  // + for lanes 0 and 3, - for the others
  return (j == 0 || j == 3) ? 1.0f : -1.0f;
}

// Eight in-place DPP multiply-adds in one asm block.  The compiler does not model the DPP
// read-after-VALU-write hazard for inline asm, so the block starts with the two wait states it
// needs; inside the block every instruction reads a register the previous two did not write.
#define TFP8_DPP_FMAC8(CTRL, a, sgn)                                                          \
  asm("s_nop 1\n\t"                                                                          \
      "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                   \
      "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                   \
      "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                   \
      "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                   \
      "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                   \
      "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                   \
      "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                   \
      "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"                         \
      : "+v"((a)[0]), "+v"((a)[1]), "+v"((a)[2]), "+v"((a)[3]), "+v"((a)[4]), "+v"((a)[5]),  \
        "+v"((a)[6]), "+v"((a)[7])                                                          \
      : "v"(sgn))

template <int N>
__device__ __forceinline__ void fwht_lanes8(float (&v)[N], int j) {
  static_assert(N % 8 == 0, "lane transform works on groups of 8 registers");
  const float s7 = (j & 4) ? -1.0f : 1.0f;
  const float s1 = (j & 1) ? -1.0f : 1.0f;
  const float s2 = (j & 2) ? -1.0f : 1.0f;
#pragma unroll
  for (int r = 0; r < N; r += 8) TFP8_DPP_FMAC8("row_half_mirror", &v[r], s7);
#pragma unroll
  for (int r = 0; r < N; r += 8) TFP8_DPP_FMAC8("quad_perm:[1,0,3,2]", &v[r], s1);
#pragma unroll
  for (int r = 0; r < N; r += 8) TFP8_DPP_FMAC8("quad_perm:[2,3,0,1]", &v[r], s2);
}

// The same over the lanes of a block of any supported width: 8 lanes as above, or 4 lanes with
// partners lane^1 and lane^2 (quad_perm), sigma from lane bits 0 and 1.  The 4-lane network
// keeps the natural order and leaves lane j with (-1)^popcount(j) * (H_4 v)[j] (enumerated on
// the unit vectors like the 8-lane one).
constexpr int lanes_per_block(int B) { return B == 64 ? 4 : 8; }

template <int L>
__device__ __forceinline__ int lane_perm(int j) {
  static_assert(L == 4 || L == 8, "4 or 8 lanes per block");
  if constexpr (L == 8) return lane8_perm(j);
  return j;
}
template <int L>
__device__ __forceinline__ float lane_sign(int j) {
  static_assert(L == 4 || L == 8, "4 or 8 lanes per block");
  if constexpr (L == 8) return lane8_sign(j);
  return (j == 0 || j == 3) ? 1.0f : -1.0f;
}
template <int L, int N>
__device__ __forceinline__ void fwht_lanes(float (&v)[N], int j) {
  static_assert(L == 4 || L == 8, "4 or 8 lanes per block");
  if constexpr (L == 8) {
    fwht_lanes8<N>(v, j);
  } else {
    const float s1 = (j & 1) ? -1.0f : 1.0f;
    const float s2 = (j & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int r = 0; r < N; r += 8) TFP8_DPP_FMAC8("quad_perm:[1,0,3,2]", &v[r], s1);
#pragma unroll
    for (int r = 0; r < N; r += 8) TFP8_DPP_FMAC8("quad_perm:[2,3,0,1]", &v[r], s2);
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// First butterfly of four packed bfloat16 pairs (one dword each): o[2q] = lo_q + hi_q and
// o[2q + 1] = lo_q - hi_q, with v_dot2_f32_bf16 against (1, 1) and (1, -1).  Each product is
// exact; the sum is rounded once (to within an ulp: the instruction does not round
// magnitude-disparate addends exactly to nearest), and bfloat16 subnormals are kept.  Written
// as asm to get the three-operand form with a zero addend (the compiler picks the accumulating
// form plus a move that zeroes the accumulator).  A DOT result must wait three states before
// another VALU instruction reads or overwrites it, and the compiler inserts those waits only
// around DOT instructions it emits itself, so the block ends with them (and starts with two,
// for inputs written just before).  Early-clobber outputs keep every result out of the
// registers of the inputs that later instructions of the block still read.
__device__ __forceinline__ void bf16_butterfly4(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3,
                                                uint32_t ones, uint32_t plus_minus, float *o) {
  asm("s_nop 1\n\t"
      "v_dot2_f32_bf16 %0, %8, %12, 0\n\t"
      "v_dot2_f32_bf16 %1, %8, %13, 0\n\t"
      "v_dot2_f32_bf16 %2, %9, %12, 0\n\t"
      "v_dot2_f32_bf16 %3, %9, %13, 0\n\t"
      "v_dot2_f32_bf16 %4, %10, %12, 0\n\t"
      "v_dot2_f32_bf16 %5, %10, %13, 0\n\t"
      "v_dot2_f32_bf16 %6, %11, %12, 0\n\t"
      "v_dot2_f32_bf16 %7, %11, %13, 0\n\t"
      "s_nop 2"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
        "=&v"(o[6]), "=&v"(o[7])
      : "v"(d0), "v"(d1), "v"(d2), "v"(d3), "v"(ones), "v"(plus_minus));
}

// acc + lo^2 + hi^2 of a packed bfloat16 pair (squares exact).
__device__ __forceinline__ float bf16_pair_sumsq(uint32_t d, float acc) {
  const bf16x2 x = __builtin_bit_cast(bf16x2, d);
  return __builtin_amdgcn_fdot2_f32_bf16(x, x, acc, false);
}

// bfloat16 pair in one dword -> two floats (exact).
__device__ __forceinline__ void widen_bf16x2(uint32_t d, float &lo, float &hi) {
  lo = __uint_as_float(d << 16);
  hi = __uint_as_float(d & 0xFFFF0000u);
}

// Four floats -> four E4M3FN bytes (OCP format, round to nearest even) in one dword.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Four E4M3FN bytes of one dword -> four floats (exact).
__device__ __forceinline__ void unpack_fp8x4(uint32_t w, float &a, float &b, float &c, float &d) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  a = lo[0];
  b = lo[1];
  c = hi[0];
  d = hi[1];
}

// INT8 codes.  fma(w, c, 1.5 * 2^23) rounds w * c to the nearest integer k (ties to even) in
// a single rounding, for |w c| < 2^22, and leaves k in the low bits of the result: the low byte
// of its bit pattern is k as a two's complement byte.
constexpr float kInt8Magic = 12582912.0f;  // 1.5 * 2^23

__device__ __forceinline__ uint32_t pack_int8x4_rounded(float a, float b, float c, float d) {
  return (__float_as_uint(a) & 0xFFu) | ((__float_as_uint(b) & 0xFFu) << 8) |
         ((__float_as_uint(c) & 0xFFu) << 16) | (__float_as_uint(d) << 24);
}

// Four INT8 codes of one dword -> four floats (exact).
__device__ __forceinline__ void unpack_int8x4(uint32_t w, float &a, float &b, float &c, float &d) {
  a = (float)(int)(int8_t)(w & 0xFFu);
  b = (float)(int)(int8_t)((w >> 8) & 0xFFu);
  c = (float)(int)(int8_t)((w >> 16) & 0xFFu);
  d = (float)((int)w >> 24);
}

__device__ __forceinline__ int exponent_of(float x) { return __builtin_amdgcn_frexp_expf(x); }
__device__ __forceinline__ float mantissa_of(float x) { return __builtin_amdgcn_frexp_mantf(x); }
__device__ __forceinline__ float scale2(float x, int k) { return __builtin_amdgcn_ldexpf(x, k); }

}  // namespace tfp8
