// tfp8_kernels.hip - gfx950 kernels for FP8 E4M3 (ASH + DS) block compression and the
// C ABI declared in include/tfp8.h.
//
// Method: page "TACO: Efficient Communication Compression of Intermediate Tensors for Scalable
// Tensor-Parallel LLM Training" (section 2.B.1 adaptive scale-Hadamard, section 2.B.2 dual
// scale, section 2.B.3 one fused kernel), and page "AGoQ: Activation and Gradient Quantization
// for Memory-Efficient Distributed Training of LLMs" (section 2.B, dequantize / FP32 sum /
// requantize).  The pages give no kernel design for this hardware; what follows is laid out
// for CDNA4 wavefronts.
//
// Layout.  A block of B elements is held by a group of 8 lanes (compress, decompress) or
// B/16 lanes (reduce).  In compress and decompress, lane j of a group holds B/8 elements as
// B/64 runs of 8 consecutive elements, run g covering elements [64g + 8j, 64g + 8j + 8) of the
// block: each 8-lane group reads or writes whole 128-byte lines of bfloat16 input.  Index bits
// 0-2 and 6.. live in registers, bits 3-5 across the 8 lanes.
//
// Transform.  w = H x (unnormalised) is computed by an in-register FWHT over the register
// bits and a 3-stage DPP butterfly over the lane bits (tfp8_device.hpp), which leaves lane j
// holding sign(j) * w at lane position perm(j).  The sign is folded into the post-scale
// multiplier and the position into the store address, so nothing is moved back.
//
// Scales.  With s = max|y|/448 and y = alpha w / sqrt(B), the codes are E4M3(448 w / max|w|)
// for every alpha (alpha cancels), so the kernel never multiplies the elements by alpha: it
// computes c = 448 / max|w|, u = w c (the codes' pre-rounding values), and gets the energy
// from sum(u^2) = c^2 sum(w^2) = c^2 B sum(x^2) (the rotation preserves energy), which stays
// inside float32 range for every block.  Then
//   alpha = clamp(c sqrt(T B^2 / sum(u^2)), 2^-126, 2^126),  s = alpha max|w| / (448 sqrt(B)).
// Blocks whose max|w| is outside [2^-100, 2^100] (bfloat16 subnormal blocks, for one) are
// first multiplied by an exact power of two and the exponent is carried into alpha and s.
//
// Reduce.  Sum of reconstructions z = sum_p H (s_p dec q_p) / (sqrt(B) alpha_p) = H r / sqrt(B)
// with r = sum_p (s_p / alpha_p) dec(q_p); requantising z gives y' = alpha' r exactly, so the
// reduce works on r directly with no Hadamard at all, and max|y'| = alpha' max|r|.  The sum is
// accumulated in float64 (as fast as unpacked float32 on this chip), which keeps it exact
// enough that contributions which largely cancel still requantise like the exact sum.

#include <math.h>
#include <stdint.h>

#include "../../include/tfp8.h"
#include "tfp8_device.hpp"

namespace tfp8 {

constexpr int kThreads = 256;  // 4 wavefronts per workgroup

// --------------------------------------------------------------------------------------------
// Shared tail: from the rotated values of one block (held by a group of L lanes) to codes,
// alpha and s.
//
//   v      values in registers; the true values are sign * v * 2^E0
//   M      max|v| over the block (every lane of the group holds it)
//   E0     exponent offset of v (0 for compress; the common exponent of the reduce)
//   TBB    T * B^2 for compress (v = H x unnormalised), T * B for reduce (v = r)
//   C      448 * sqrt(B) for compress, 448 for reduce
//   sign   +-1 lane sign folded into the code multiplier
// Outputs u[] (pre-rounding code values) and the block's alpha and s.
template <int L, int N>
__device__ __forceinline__ void requant_tail(float (&v)[N], float M, int E0, float TBB, float C,
                                             float sign, float &alpha_out, float &scale_out) {
  int E = E0;
  if (M != 0.0f && !(M >= 0x1p-100f && M <= 0x1p100f)) {
    // Bring max|v| into [1, 2) by an exact power of two so that 448 / M is a normal float.
    const int k = 1 - exponent_of(M);
#pragma unroll
    for (int r = 0; r < N; ++r) v[r] = scale2(v[r], k);
    M = scale2(M, k);
    E -= k;
  }
  const bool zero = (M == 0.0f);
  const float c = zero ? 0.0f : __fdiv_rn(448.0f, M);
  const float cl = c * sign;
  float su = 0.0f;
#pragma unroll
  for (int r = 0; r < N; ++r) {
    v[r] = fmaf(v[r], cl, 0.0f);  // + 0 turns a -0 product into +0
    su = fmaf(v[r], v[r], su);
  }
  const float SU = group_sum<L>(su);
  const float a2 = c * __fsqrt_rn(__fdiv_rn(TBB, SU));
  const float alpha = fminf(fmaxf(scale2(a2, -E), 0x1p-126f), 0x1p126f);
  const float s = __fdiv_rn(scale2(alpha, E) * M, C);
  alpha_out = zero ? 1.0f : alpha;
  scale_out = zero ? 0.0f : s;
}

// --------------------------------------------------------------------------------------------
// K1: compress.  One wavefront handles 8 blocks per iteration of a grid-stride loop.

template <int B, bool F32IN>
__global__ __launch_bounds__(kThreads) void k_compress(const void *__restrict__ xin, int64_t nb,
                                                       float TBB, float C,
                                                       uint8_t *__restrict__ codes,
                                                       float *__restrict__ alpha_out,
                                                       float *__restrict__ scale_out) {
  constexpr int N = B / 8;   // elements per lane
  constexpr int G = N / 8;   // runs of 8 consecutive elements per lane
  const int lane = threadIdx.x & 63;
  const int j = lane & 7;
  const int bw = lane >> 3;
  const int pj = lane8_perm(j);
  const float sj = lane8_sign(j);
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t ntiles = (nb + 7) >> 3;

  for (int64_t tile = wave; tile < ntiles; tile += nwaves) {
    const int64_t blk = tile * 8 + bw;
    const bool active = blk < nb;
    float v[N];
    if (active) {
      if constexpr (!F32IN) {
        const uint16_t *xb = (const uint16_t *)xin + blk * B + 8 * j;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const u32x4 d = *(const u32x4 *)(xb + 64 * g);
#pragma unroll
          for (int q = 0; q < 4; ++q) widen_bf16x2(d[q], v[8 * g + 2 * q], v[8 * g + 2 * q + 1]);
        }
      } else {
        const float *xb = (const float *)xin + blk * B + 8 * j;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const u32x4 d0 = *(const u32x4 *)(xb + 64 * g);
          const u32x4 d1 = *(const u32x4 *)(xb + 64 * g + 4);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[8 * g + q] = __uint_as_float(d0[q]);
            v[8 * g + 4 + q] = __uint_as_float(d1[q]);
          }
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < N; ++r) v[r] = 0.0f;
    }

    // orthogonal Hadamard rotation (unnormalised; 1/sqrt(B) and alpha are carried in s)
    fwht_registers<N>(v);
    fwht_lanes8<N>(v, j);

    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < N; ++r) m = fmaxf(m, fabsf(v[r]));
    const float M = group_max<8>(m);

    float alpha, s;
    requant_tail<8, N>(v, M, 0, TBB, C, sj, alpha, s);

    if (active) {
      uint8_t *cb = codes + blk * B + 8 * pj;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        u32x2 w;
        w[0] = pack_fp8x4(v[8 * g + 0], v[8 * g + 1], v[8 * g + 2], v[8 * g + 3]);
        w[1] = pack_fp8x4(v[8 * g + 4], v[8 * g + 5], v[8 * g + 6], v[8 * g + 7]);
        *(u32x2 *)(cb + 64 * g) = w;
      }
      if (j == 0) {
        alpha_out[blk] = alpha;
        scale_out[blk] = s;
      }
    }
  }
}

// --------------------------------------------------------------------------------------------
// K2: decompress.  x = H (s dec q) / (sqrt(B) alpha), same lane layout as compress.

template <int B, bool F32OUT>
__global__ __launch_bounds__(kThreads) void k_decompress(const uint8_t *__restrict__ codes,
                                                         const float *__restrict__ alpha,
                                                         const float *__restrict__ scale,
                                                         int64_t nb, float inv_sqrt_b,
                                                         void *__restrict__ out) {
  constexpr int N = B / 8;
  constexpr int G = N / 8;
  const int lane = threadIdx.x & 63;
  const int j = lane & 7;
  const int bw = lane >> 3;
  const int pj = lane8_perm(j);
  const float sj = lane8_sign(j);
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t ntiles = (nb + 7) >> 3;

  for (int64_t tile = wave; tile < ntiles; tile += nwaves) {
    const int64_t blk = tile * 8 + bw;
    const bool active = blk < nb;
    float v[N];
    float s = 0.0f, a = 1.0f;
    if (active) {
      const uint8_t *cb = codes + blk * B + 8 * j;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const u32x2 w = *(const u32x2 *)(cb + 64 * g);
        unpack_fp8x4(w[0], v[8 * g + 0], v[8 * g + 1], v[8 * g + 2], v[8 * g + 3]);
        unpack_fp8x4(w[1], v[8 * g + 4], v[8 * g + 5], v[8 * g + 6], v[8 * g + 7]);
      }
      s = scale[blk];
      a = alpha[blk];
    } else {
#pragma unroll
      for (int r = 0; r < N; ++r) v[r] = 0.0f;
    }

    // The decoded values are multiples of 2^-9 below 2^8.81, so every partial sum of the
    // transform is exact in float32 until it passes 2^15 (for B <= 128 only the last stage
    // can round, once).
    fwht_registers<N>(v);
    fwht_lanes8<N>(v, j);

    // (v * s / sqrt(B)) / alpha as two products: s / (sqrt(B) alpha) alone can fall below the
    // normal range when alpha is large, the two-step form only rounds the final value there.
    const float f = (s == 0.0f) ? 0.0f : sj * (s * inv_sqrt_b);
    const float ra = __frcp_rn(a);

    if (active) {
      if constexpr (F32OUT) {
        float *ob = (float *)out + blk * B + 8 * pj;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          u32x4 w0, w1;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            w0[q] = __float_as_uint(fmaf(v[8 * g + q], f, 0.0f) * ra);
            w1[q] = __float_as_uint(fmaf(v[8 * g + 4 + q], f, 0.0f) * ra);
          }
          *(u32x4 *)(ob + 64 * g) = w0;
          *(u32x4 *)(ob + 64 * g + 4) = w1;
        }
      } else {
        __bf16 *ob = (__bf16 *)out + blk * B + 8 * pj;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          u32x4 w;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const __bf16 lo = (__bf16)(fmaf(v[8 * g + 2 * q], f, 0.0f) * ra);
            const __bf16 hi = (__bf16)(fmaf(v[8 * g + 2 * q + 1], f, 0.0f) * ra);
            w[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          }
          *(u32x4 *)(ob + 64 * g) = w;
        }
      }
    }
  }
}

// --------------------------------------------------------------------------------------------
// K3: reduce.  B/16 lanes per block, 16 consecutive codes per lane (one 16-byte load per
// contribution), no Hadamard.

template <int B>
__global__ __launch_bounds__(kThreads) void k_reduce(const uint8_t *__restrict__ codes,
                                                     const float *__restrict__ alpha,
                                                     const float *__restrict__ scale, int P,
                                                     int64_t n, int64_t nb, float TB,
                                                     uint8_t *__restrict__ codes_out,
                                                     float *__restrict__ alpha_out,
                                                     float *__restrict__ scale_out) {
  constexpr int L = B / 16;    // lanes per block
  constexpr int BPW = 64 / L;  // blocks per wavefront
  const int lane = threadIdx.x & 63;
  const int j = lane % L;
  const int bw = lane / L;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t ntiles = (nb + BPW - 1) / BPW;

  for (int64_t tile = wave; tile < ntiles; tile += nwaves) {
    const int64_t blk = tile * BPW + bw;
    const bool active = blk < nb;
    const int64_t cblk = active ? blk : 0;  // inactive groups read block 0 and store nothing

    // Common exponent of the dequantisation factors g_p = s_p / alpha_p: every g_p is
    // divided by 2^Emax so that the largest is near 1 and the sum rounds to a normal float32.
    int Emax = -100000;
    for (int p = 0; p < P; ++p) {
      const float sp = scale[(int64_t)p * nb + cblk];
      const float ap = alpha[(int64_t)p * nb + cblk];
      if (sp != 0.0f) Emax = max(Emax, exponent_of(sp) - exponent_of(ap));
    }
    if (Emax == -100000) Emax = 0;

    // r = sum_p g_p dec(q_p), accumulated in float64.  g_p is cut to 49 significant bits
    // (a relative change below 2^-48), so that its product with an E4M3 value (at most 4
    // significant bits) is exact in float64; the only roundings are those of the running sum,
    // each within 2^-53 of it.  Contributions that largely cancel therefore still requantise
    // like the exact sum, and a contribution and its exact negation cancel to exactly zero.
    double r64[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) r64[i] = 0.0;
    const uint8_t *cb = codes + cblk * B + 16 * j;
    for (int p = 0; p < P; ++p) {
      const float sp = scale[(int64_t)p * nb + cblk];
      const float ap = alpha[(int64_t)p * nb + cblk];
      double g = (sp == 0.0f) ? 0.0 : __builtin_amdgcn_ldexp((double)sp / (double)ap, -Emax);
      g = __longlong_as_double(__double_as_longlong(g) & ~0xFLL);
      const u32x4 d = *(const u32x4 *)(cb + (int64_t)p * n);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float a0, a1, a2, a3;
        unpack_fp8x4(d[q], a0, a1, a2, a3);
        r64[4 * q + 0] = fma((double)a0, g, r64[4 * q + 0]);
        r64[4 * q + 1] = fma((double)a1, g, r64[4 * q + 1]);
        r64[4 * q + 2] = fma((double)a2, g, r64[4 * q + 2]);
        r64[4 * q + 3] = fma((double)a3, g, r64[4 * q + 3]);
      }
    }

    float r[16];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      r[i] = (float)r64[i];
      m = fmaxf(m, fabsf(r[i]));
    }
    float M = group_max<L>(m);
    int E = Emax;
    if (M != 0.0f && !(M >= 0x1p-100f && M <= 0x1p100f)) {
      // The contributions cancelled (or all were tiny): rescale the float64 sum so that its
      // largest magnitude lies in [1, 2) before rounding it to float32.
      double m64 = 0.0;
#pragma unroll
      for (int i = 0; i < 16; ++i) m64 = fmax(m64, fabs(r64[i]));
      const int e64 = __builtin_amdgcn_frexp_exp(m64);
      const int k = 1 - group_max_i<L>(e64);
      m = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        r[i] = (float)__builtin_amdgcn_ldexp(r64[i], k);
        m = fmaxf(m, fabsf(r[i]));
      }
      M = group_max<L>(m);
      E -= k;
    }

    // the true sum is r * 2^E
    float a_out, s_out;
    requant_tail<L, 16>(r, M, E, TB, 448.0f, 1.0f, a_out, s_out);
    if (active) {
      u32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = pack_fp8x4(r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3]);
      *(u32x4 *)(codes_out + blk * B + 16 * j) = w;
      if (j == 0) {
        alpha_out[blk] = a_out;
        scale_out[blk] = s_out;
      }
    }
  }
}

}  // namespace tfp8

// ============================================================================================
// Host side of the C ABI: argument checks (before any HIP call), kernel choice, launch shape.

namespace {

using namespace tfp8;

bool block_ok(int32_t block) {
  return block == 64 || block == 128 || block == 256 || block == 512;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void *p, int64_t bytes) {
  return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool target_ok(float t) {
  return isfinite(t) && t >= 0x1p-64f && t <= 0x1p64f;
}

// Workgroups for a grid-stride launch: one wavefront per tile up to 8 resident workgroups
// (32 wavefronts) per compute unit.
unsigned grid_for(int64_t tiles) {
  static int cu_count = 0;
  if (cu_count == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0)
      cu_count = cus;
    else
      cu_count = 256;
  }
  const int64_t wgs = (tiles + (kThreads / 64) - 1) / (kThreads / 64);
  const int64_t cap = (int64_t)cu_count * 8;
  return (unsigned)(wgs < cap ? (wgs > 0 ? wgs : 1) : cap);
}

tfp8_status launched() {
  return hipGetLastError() == hipSuccess ? TFP8_OK : TFP8_E_HIP;
}

template <int B>
tfp8_status launch_compress(const void *x, bool f32, int64_t nb, float target, uint8_t *codes,
                            float *alpha, float *scale, hipStream_t st) {
  const float TBB = target * (float)B * (float)B;  // exact: powers of two
  const float C = (float)(448.0 * sqrt((double)B));
  const unsigned grid = grid_for((nb + 7) / 8);
  if (f32)
    hipLaunchKernelGGL((k_compress<B, true>), dim3(grid), dim3(kThreads), 0, st, x, nb, TBB, C,
                       codes, alpha, scale);
  else
    hipLaunchKernelGGL((k_compress<B, false>), dim3(grid), dim3(kThreads), 0, st, x, nb, TBB, C,
                       codes, alpha, scale);
  return launched();
}

template <int B>
tfp8_status launch_decompress(const uint8_t *codes, const float *alpha, const float *scale,
                              int64_t nb, void *out, bool f32, hipStream_t st) {
  const float inv_sqrt_b = (float)(1.0 / sqrt((double)B));
  const unsigned grid = grid_for((nb + 7) / 8);
  if (f32)
    hipLaunchKernelGGL((k_decompress<B, true>), dim3(grid), dim3(kThreads), 0, st, codes, alpha,
                       scale, nb, inv_sqrt_b, out);
  else
    hipLaunchKernelGGL((k_decompress<B, false>), dim3(grid), dim3(kThreads), 0, st, codes, alpha,
                       scale, nb, inv_sqrt_b, out);
  return launched();
}

template <int B>
tfp8_status launch_reduce(const uint8_t *codes, const float *alpha, const float *scale, int P,
                          int64_t n, int64_t nb, float target, uint8_t *codes_out,
                          float *alpha_out, float *scale_out, hipStream_t st) {
  const float TB = target * (float)B;
  constexpr int BPW = 64 / (B / 16);
  const unsigned grid = grid_for((nb + BPW - 1) / BPW);
  hipLaunchKernelGGL((k_reduce<B>), dim3(grid), dim3(kThreads), 0, st, codes, alpha, scale, P, n,
                     nb, TB, codes_out, alpha_out, scale_out);
  return launched();
}

}  // namespace

extern "C" {

int32_t tfp8_version(void) { return (1 << 16) | 0; }

const char *tfp8_status_string(tfp8_status status) {
  switch (status) {
    case TFP8_OK: return "ok";
    case TFP8_E_NULL: return "a required pointer is NULL";
    case TFP8_E_SIZE: return "n is negative or not a multiple of the block size";
    case TFP8_E_BLOCK: return "unsupported block size (use 64, 128, 256 or 512)";
    case TFP8_E_DTYPE: return "unsupported dtype (use TFP8_BF16 or TFP8_F32)";
    case TFP8_E_ALIGN: return "misaligned pointer (16 bytes for data, 4 for scales)";
    case TFP8_E_ARG: return "bad argument (P, target, or overlapping buffers)";
    case TFP8_E_HIP: return "the HIP runtime rejected the kernel launch";
  }
  return "unknown status";
}

tfp8_status tfp8_compress(const void *x, tfp8_dtype x_dtype, int64_t n, int32_t block, float target,
                          uint8_t *codes, float *alpha, float *scale, void *stream) {
  if (!block_ok(block)) return TFP8_E_BLOCK;
  if (n < 0 || n % block != 0) return TFP8_E_SIZE;
  if (x_dtype != TFP8_BF16 && x_dtype != TFP8_F32) return TFP8_E_DTYPE;
  if (!target_ok(target)) return TFP8_E_ARG;
  if (n == 0) return TFP8_OK;
  if (!x || !codes || !alpha || !scale) return TFP8_E_NULL;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(alpha, 4) || !aligned(scale, 4))
    return TFP8_E_ALIGN;
  const int64_t nb = n / block;
  const Range rx = range_of(x, n * (x_dtype == TFP8_F32 ? 4 : 2)), rc = range_of(codes, n),
              ra = range_of(alpha, nb * 4), rs = range_of(scale, nb * 4);
  if (overlap(rx, rc) || overlap(rx, ra) || overlap(rx, rs) || overlap(rc, ra) ||
      overlap(rc, rs) || overlap(ra, rs))
    return TFP8_E_ARG;
  hipStream_t st = (hipStream_t)stream;
  const bool f32 = x_dtype == TFP8_F32;
  switch (block) {
    case 64: return launch_compress<64>(x, f32, nb, target, codes, alpha, scale, st);
    case 128: return launch_compress<128>(x, f32, nb, target, codes, alpha, scale, st);
    case 256: return launch_compress<256>(x, f32, nb, target, codes, alpha, scale, st);
    default: return launch_compress<512>(x, f32, nb, target, codes, alpha, scale, st);
  }
}

tfp8_status tfp8_decompress(const uint8_t *codes, const float *alpha, const float *scale, int64_t n,
                            int32_t block, void *out, tfp8_dtype out_dtype, void *stream) {
  if (!block_ok(block)) return TFP8_E_BLOCK;
  if (n < 0 || n % block != 0) return TFP8_E_SIZE;
  if (out_dtype != TFP8_BF16 && out_dtype != TFP8_F32) return TFP8_E_DTYPE;
  if (n == 0) return TFP8_OK;
  if (!codes || !alpha || !scale || !out) return TFP8_E_NULL;
  if (!aligned(out, 16) || !aligned(codes, 16) || !aligned(alpha, 4) || !aligned(scale, 4))
    return TFP8_E_ALIGN;
  const int64_t nb = n / block;
  const Range ro = range_of(out, n * (out_dtype == TFP8_F32 ? 4 : 2));
  if (overlap(ro, range_of(codes, n)) || overlap(ro, range_of(alpha, nb * 4)) ||
      overlap(ro, range_of(scale, nb * 4)))
    return TFP8_E_ARG;
  hipStream_t st = (hipStream_t)stream;
  const bool f32 = out_dtype == TFP8_F32;
  switch (block) {
    case 64: return launch_decompress<64>(codes, alpha, scale, nb, out, f32, st);
    case 128: return launch_decompress<128>(codes, alpha, scale, nb, out, f32, st);
    case 256: return launch_decompress<256>(codes, alpha, scale, nb, out, f32, st);
    default: return launch_decompress<512>(codes, alpha, scale, nb, out, f32, st);
  }
}

tfp8_status tfp8_reduce_fp8(const uint8_t *codes, const float *alpha, const float *scale, int32_t P,
                            int64_t n, int32_t block, float target, uint8_t *codes_out,
                            float *alpha_out, float *scale_out, void *stream) {
  if (!block_ok(block)) return TFP8_E_BLOCK;
  if (n < 0 || n % block != 0) return TFP8_E_SIZE;
  if (P < 1 || P > 64 || !target_ok(target)) return TFP8_E_ARG;
  if (n == 0) return TFP8_OK;
  if (!codes || !alpha || !scale || !codes_out || !alpha_out || !scale_out) return TFP8_E_NULL;
  if (!aligned(codes, 16) || !aligned(codes_out, 16) || !aligned(alpha, 4) || !aligned(scale, 4) ||
      !aligned(alpha_out, 4) || !aligned(scale_out, 4))
    return TFP8_E_ALIGN;
  const int64_t nb = n / block;
  const Range ins[3] = {range_of(codes, (int64_t)P * n), range_of(alpha, (int64_t)P * nb * 4),
                        range_of(scale, (int64_t)P * nb * 4)};
  const Range outs[3] = {range_of(codes_out, n), range_of(alpha_out, nb * 4),
                         range_of(scale_out, nb * 4)};
  for (int i = 0; i < 3; ++i) {
    for (int k = 0; k < 3; ++k)
      if (overlap(outs[i], ins[k])) return TFP8_E_ARG;
    for (int k = i + 1; k < 3; ++k)
      if (overlap(outs[i], outs[k])) return TFP8_E_ARG;
  }
  hipStream_t st = (hipStream_t)stream;
  switch (block) {
    case 64: return launch_reduce<64>(codes, alpha, scale, P, n, nb, target, codes_out, alpha_out, scale_out, st);
    case 128: return launch_reduce<128>(codes, alpha, scale, P, n, nb, target, codes_out, alpha_out, scale_out, st);
    case 256: return launch_reduce<256>(codes, alpha, scale, P, n, nb, target, codes_out, alpha_out, scale_out, st);
    default: return launch_reduce<512>(codes, alpha, scale, P, n, nb, target, codes_out, alpha_out, scale_out, st);
  }
}

}  // extern "C"
