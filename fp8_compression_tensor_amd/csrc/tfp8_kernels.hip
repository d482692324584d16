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
// Layout.  A block of B elements is held by a group of L lanes (compress: L = 8, with a pair
// of blocks per group at B = 64; accumulate: L = 8, or 4 at B = 64 so that a lane still holds
// 16 elements; decompress: L = 8) or B/16 lanes (reduce).  In the L-lane kernels lane j of a
// group holds B/L elements as runs of 8 consecutive elements, run g covering elements
// [8Lg + 8j, 8Lg + 8j + 8) of the block: each group reads or writes whole runs of 8L
// consecutive elements.  At L = 8 index bits 0-2 and 6.. live in registers, bits 3-5 across the
// lanes (at B = 64 in compress, run g is block g of the pair).  float32 data (compress's input,
// decompress's output, accumulate's gradient at 8 lanes per block) takes another assignment
// within each run of 64: lane j holds [4 j, 4 j + 4) and [32 + 4 j, 32 + 4 j + 4), so that each
// 16-byte access instruction of a group covers whole lines (see load_compress_at).
//
// Launch.  One tile (64/L blocks) per wavefront, 8- or 16-byte vector loads and stores per
// lane, no LDS, no atomics.  Compress of an input of 1.5 GiB or more launches
// one-wavefront workgroups and gives each XCD a contiguous eighth of the tiles
// (kCompressRemapMinBytes below).
//
// Transform.  w = H x (unnormalised) is computed by an in-register FWHT over the register
// bits and a 3-stage DPP butterfly over the lane bits (tfp8_device.hpp), which leaves lane j
// holding sign(j) * w at lane position perm(j).  The sign is folded into the post-scale
// multiplier and the position into the store address, so nothing is moved back.
//
// Scales.  With s = max|y|/448 and y = alpha w / sqrt(B), the codes are E4M3(448 w / max|w|)
// for every alpha (alpha cancels), so the kernel never multiplies the elements by alpha: it
// computes c = 448 / max|w| and u = w c (the codes' pre-rounding values), takes the energy
// sum(x^2) straight from the packed input, and sets
//   alpha = clamp(sqrt(T B / sum(x^2)), 2^-126, 2^126),  s = alpha max|w| / (448 sqrt(B)).
// For blocks whose max|w| is outside [2^-40, 2^60] compress stores an all-zero block directly
// and brings a bfloat16-subnormal or huge block into range by an exact power of two, taking the
// energy from the scaled w (the rotation preserves energy); the reduce and the accumulation use
// scales_exact, which does the same for sums whose range it cannot bound in advance.
//
// Reduce.  Sum of reconstructions z = sum_p H (s_p dec q_p) / (sqrt(B) alpha_p) = H r / sqrt(B)
// with r = sum_p (s_p / alpha_p) dec(q_p); requantising z gives y' = alpha' r exactly, so the
// reduce works on r directly with no Hadamard at all, and max|y'| = alpha' max|r|.  The sum is
// accumulated in float64 (as fast as unpacked float32 on this chip), which keeps it exact
// enough that contributions which cancel down to about 2^-25 of their peaks still requantise
// like the exact sum (below that, a float64 sum's rounding noise is what remains).
//
// Accumulate (AGoQ page, section 2.B, local accumulation).  A compressed main gradient plus a
// dense local gradient, requantised, also in the rotated domain: only the local gradient is
// transformed.  Blocks where the two cancel are redone by a second kernel with an exact split
// of the transform (K4 below).
//
// Variants.  Every kernel is a template on FLAGS: INT8 codes (Q_max = 127, the TACO page's INT8
// fallback, section 5) and the rotation left out (ablation), alone or together.

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <tuple>

#include "../../include/tfp8.h"
#include "tfp8_device.hpp"

namespace tfp8 {

constexpr int kThreads = 256;  // 4 wavefronts per workgroup (compress: 1 or 4, see its launch)

// Index of this wavefront among the launch's, for a launch of `wpw` wavefronts per workgroup
// (passed as an argument: blockDim would be read from the dispatch packet with a memory load at
// the start of every wavefront).  With `remap`, workgroup b, which the dispatcher hands to XCD
// b mod 8 in round robin, takes the slot (b mod 8) * gridDim.x / 8 + b / 8, so that each XCD
// streams one contiguous eighth of the tiles (the host then launches a multiple of 8
// workgroups).
__device__ __forceinline__ int64_t wave_index(int wpw, bool remap) {
  int64_t b = blockIdx.x;
  if (remap) b = (b & 7) * (int64_t)(gridDim.x >> 3) + (b >> 3);
  return b * wpw + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

// Variant bits of the *_ex entry points, as compile-time kernel parameters.
constexpr int kInt8 = 1;        // INT8 codes, Q_max = 127 (else E4M3, Q_max = 448)
constexpr int kNoRotation = 2;  // leave the Hadamard out (ablation)

template <int FLAGS>
constexpr float qmax_of() { return (FLAGS & kInt8) ? 127.0f : 448.0f; }

// Codes of four values v * cm (cm: code multiplier with any lane sign folded in).
template <int FLAGS>
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d, float cm) {
  if constexpr (FLAGS & kInt8) {
    return pack_int8x4_rounded(fmaf(a, cm, kInt8Magic), fmaf(b, cm, kInt8Magic),
                               fmaf(c, cm, kInt8Magic), fmaf(d, cm, kInt8Magic));
  } else {
    // + 0 turns a -0 product into +0
    return pack_fp8x4(fmaf(a, cm, 0.0f), fmaf(b, cm, 0.0f), fmaf(c, cm, 0.0f), fmaf(d, cm, 0.0f));
  }
}

template <int FLAGS>
__device__ __forceinline__ void decode4(uint32_t w, float &a, float &b, float &c, float &d) {
  if constexpr (FLAGS & kInt8)
    unpack_int8x4(w, a, b, c, d);
  else
    unpack_fp8x4(w, a, b, c, d);
}

// Streaming loads and stores: every input byte is read once and every output byte written
// once, so they carry the non-temporal hint.  (Plain accesses measure faster when the caches
// are flushed between single launches, because the output then waits in the 256 MB MALL and
// its write to HBM falls outside the launch; over back-to-back launches that rotate through
// more buffers than the caches hold, where every write is paid, the hints are 4-13% faster for
// compress and decompress on 34-117 M-element inputs.)
template <class T>
__device__ __forceinline__ T ld_stream(const T *p) {
  return __builtin_nontemporal_load(p);
}
template <class T>
__device__ __forceinline__ void st_stream(T v, T *p) {
  __builtin_nontemporal_store(v, p);
}

// Codes of NR runs of 64 elements held in the float32 line layout (lane pj: elements
// [4 pj, 4 pj + 4) of each run in registers 8 t .. 8 t + 3 of v, [32 + 4 pj, 32 + 4 pj + 4) in
// 8 t + 4 .. 8 t + 7), stored from run0 on (run t at run0 + RS t).  The two code words of a run
// (A_pj, B_pj) are not contiguous; lanes pj = 2m and 2m + 1 swap one, so that the even lane
// stores A_2m A_2m+1 at 8 m and the odd lane B_2m B_2m+1 at 32 + 8 m: 8 contiguous bytes each,
// every byte of the run once.  The partner (pj ^ 1) is lane j ^ 5 under the lane network's
// permutation (lane j ^ 1 without the rotation); ds_swizzle reads it (and-mask 31, xor-mask 5 or
// 1) within the same group of 8 lanes, so under a branch taken by whole groups a lane never
// reads an inactive one.  All of the swaps are issued before the stores, so that one wait covers
// them (interleaved, they were slower than no swap at B = 512).
template <int FLAGS, int NR, int RS, bool ROT>
__device__ __forceinline__ void store_codes_line(const float *v, float cm, int pj,
                                                 uint8_t *run0) {
  const bool odd = pj & 1;
  u32x2 o[NR];
#pragma unroll
  for (int t = 0; t < NR; ++t) {
    const uint32_t wa = encode4<FLAGS>(v[8 * t + 0], v[8 * t + 1], v[8 * t + 2], v[8 * t + 3], cm);
    const uint32_t wb = encode4<FLAGS>(v[8 * t + 4], v[8 * t + 5], v[8 * t + 6], v[8 * t + 7], cm);
    const uint32_t got = __builtin_amdgcn_ds_swizzle(odd ? wa : wb, ROT ? 0x141F : 0x041F);
    o[t][0] = odd ? got : wa;
    o[t][1] = odd ? wb : got;
  }
  uint8_t *p = run0 + (odd ? 32 + 4 * (pj - 1) : 4 * pj);
#pragma unroll
  for (int t = 0; t < NR; ++t) st_stream(o[t], (u32x2 *)(p + RS * t));
}

// --------------------------------------------------------------------------------------------
// Range-safe scales: from the rotated values of one block (held by a group of L lanes) to the
// code multiplier, alpha and s, for any block -- all-zero, bfloat16-subnormal or huge.
//
//   v      values in registers; the true values are v * 2^E0 (times the lane sign)
//   M      max|v| over the block (every lane of the group holds it)
//   E0     exponent offset of v (0 for compress; the reduce's common exponent)
//   TBB    T * B^2 for compress (v = H x unnormalised), T * B for reduce and for compress
//          without the rotation (v = r or v = x)
//   Q      Q_max (448 for E4M3 codes, 127 for INT8 codes)
//   C      Q * sqrt(B) for compress, Q for reduce and for compress without the rotation
//   sign   +-1 lane sign folded into the code multiplier
// On return v may be rescaled by a power of two, and v * code_mult are the codes' values.
template <int L, int N>
__device__ __forceinline__ void scales_exact(float (&v)[N], float M, int E0, float TBB, float Q,
                                             float C, float sign, float &code_mult,
                                             float &alpha_out, float &scale_out) {
  int E = E0;
  if (M != 0.0f && !(M >= 0x1p-100f && M <= 0x1p100f)) {
    // Bring max|v| into [1, 2) by an exact power of two so that Q / M is a normal float.
    const int k = 1 - exponent_of(M);
#pragma unroll
    for (int r = 0; r < N; ++r) v[r] = scale2(v[r], k);
    M = scale2(M, k);
    E -= k;
  }
  const bool zero = (M == 0.0f);
  const float c = zero ? 0.0f : __fdiv_rn(Q, M);
  // energy from the codes' values u = v c: sum(u^2) = c^2 sum(v^2) stays in float32 range
  const float SU = group_sum<L>(sum_squares<N, true>(v, c));
  const float a2 = c * __fsqrt_rn(__fdiv_rn(TBB, SU));
  const float alpha = fminf(fmaxf(scale2(a2, -E), 0x1p-126f), 0x1p126f);
  const float s = __fdiv_rn(scale2(alpha, E) * M, C);
  code_mult = c * sign;
  alpha_out = zero ? 1.0f : alpha;
  scale_out = zero ? 0.0f : s;
}

// --------------------------------------------------------------------------------------------
// K1: compress.  One wavefront handles a tile of 8 lane groups (8 blocks, or 16 at B = 64): one
// tile per wavefront, or (LOOP, for capped launches) a tile per iteration of a grid-stride loop
// that prefetches the next iteration's input before working on the current one.

template <int B, bool F32IN>
struct CompressIn {
  static constexpr int kRuns = B / (8 * lanes_per_block(B));  // 8-element runs per lane
  static constexpr int kLoads = F32IN ? 2 * kRuns : kRuns;      // 16-byte loads per lane
  u32x4 d[kLoads];
};

// Lane j of a block's group holds the runs of 8 elements [RS g + 8 j, RS g + 8 j + 8) of its
// block, where RS = 8 L is the run stride for L lanes per block.  Compress reads them from
// the base of a tile (wave-uniform, so it stays in scalar registers) and a lane's 32-bit
// element offset into it: the loads then take the scalar base plus a vector offset, and no
// 64-bit address arithmetic runs per lane.  Run g is read at off + g * step.
//
// float32 input takes a different element-to-lane assignment within each run of 64: lane j
// holds [4 j, 4 j + 4) and [32 + 4 j, 32 + 4 j + 4) (lane bits = element bits 2-4, register bit
// 2 = element bit 5), so that each of its two 16-byte loads per run reads whole lines across the
// group; with 8 consecutive floats per lane each load instruction read half of every line.  The
// transform is the same under any assignment used for both input and output (H[i][k] =
// (-1)^popcount(i & k) is unchanged when one permutation of the bits is applied to i and k), so
// only the addresses change; the codes then come out as two 4-byte words per run, which partner
// lanes exchange to store 8 contiguous bytes each (see the store).  With the exchange, float32
// compress ran 7-11% faster over rotating buffers at every B (117 M elements: 94.6 against
// 102.6 us at B = 128, 99.0 against 105.6 us at B = 512; 470 M elements at B = 128: 380.9
// against 419.0 us).
template <bool F32IN>
constexpr int compress_lane_elems() { return F32IN ? 4 : 8; }  // a lane's first run: [c j, c j + c)
template <int B, bool F32IN>
__device__ __forceinline__ void load_compress_at(CompressIn<B, F32IN> &in, const void *tile,
                                                 uint32_t off, uint32_t step) {
  constexpr int G = CompressIn<B, F32IN>::kRuns;
  if constexpr (!F32IN) {
    const uint16_t *xb = (const uint16_t *)tile + off;
#pragma unroll
    for (int g = 0; g < G; ++g) in.d[g] = ld_stream((const u32x4 *)(xb + step * g));
  } else {
    const float *xb = (const float *)tile + off;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      in.d[2 * g] = ld_stream((const u32x4 *)(xb + step * g));
      in.d[2 * g + 1] = ld_stream((const u32x4 *)(xb + step * g + 32));
    }
  }
}

// Runs of 8 consecutive elements of block blk for either input type (lane j: [RS g + 8 j,
// RS g + 8 j + 8)): the layout of accumulate at 4 lanes per block, and of its fix pass.
template <int B, bool F32IN>
__device__ __forceinline__ void load_compress_in(CompressIn<B, F32IN> &in, const void *xin,
                                                 int64_t blk, int j) {
  constexpr int RS = 8 * lanes_per_block(B);
  constexpr int G = CompressIn<B, F32IN>::kRuns;
  if constexpr (!F32IN) {
    const uint16_t *xb = (const uint16_t *)xin + blk * B + 8 * j;
#pragma unroll
    for (int g = 0; g < G; ++g) in.d[g] = ld_stream((const u32x4 *)(xb + RS * g));
  } else {
    const float *xb = (const float *)xin + blk * B + 8 * j;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      in.d[2 * g] = ld_stream((const u32x4 *)(xb + RS * g));
      in.d[2 * g + 1] = ld_stream((const u32x4 *)(xb + RS * g + 4));
    }
  }
}

// Compress keeps 8 lanes per group at every B.  At B = 64 a group holds a pair of adjacent
// blocks, one per 64-element run (lane j: elements [8 j, 8 j + 8) of each), so that its loads
// and stores cover whole 128-byte lines exactly as at B = 128; the transform, the statistics and
// the scales are then taken per run.  (With 4 lanes per block each load instruction read half a
// line and each store wrote 32 bytes: 524 us, 70% of HBM peak, against 485 us with the pair
// layout on 8 stacked 117 M-element shards.)
constexpr int compress_blocks_per_group(int B) { return B == 64 ? 2 : 1; }

// LOOP = false: the launch has a wavefront for every tile (the host checks), so each wavefront
// takes one tile and carries no prefetch buffer, which at B = 256 leaves registers for eight
// wavefronts per SIMD instead of five.  LOOP = true: grid-stride loop with the next tile's loads
// in flight, for launches capped below one wavefront per tile (past 2^27 B elements, 2^34 at
// B = 64).
template <int B, bool F32IN, int FLAGS, bool LOOP>
__global__ __launch_bounds__(kThreads) void k_compress(const void *__restrict__ xin, int64_t nb,
                                                       float TBB, float sqrtTB, float C,
                                                       float invC, uint8_t *__restrict__ codes,
                                                       float *__restrict__ alpha_out,
                                                       float *__restrict__ scale_out, int wpw,
                                                       bool remap) {
  constexpr int L = 8;                                  // lanes per group
  constexpr int BG = compress_blocks_per_group(B);      // blocks per group (one per run at 2)
  constexpr int BPW = 64 / L * BG;                      // blocks per wavefront (one tile)
  constexpr int RS = 8 * L;                             // run stride
  constexpr int N = B * BG / L;                         // elements per lane
  constexpr int G = N / 8;                              // runs of 8 consecutive elements per lane
  constexpr int NB = N / BG;                            // a block's registers in a lane
  static_assert(CompressIn<B, F32IN>::kRuns == G, "compress input layout");
  constexpr bool ROT = !(FLAGS & kNoRotation);
  constexpr float Q = qmax_of<FLAGS>();
  const int lane = threadIdx.x & 63;
  const int j = lane & (L - 1);
  const int bw = lane / L;
  const int pj = ROT ? lane_perm<L>(j) : j;
  const float sj = ROT ? lane_sign<L>(j) : 1.0f;
  const int64_t wave = wave_index(wpw, remap);
  const int64_t nwaves = (int64_t)gridDim.x * wpw;
  const int64_t ntiles = (int64_t)(((uint64_t)nb + BPW - 1) / BPW);  // nb >= 0
  // packed bfloat16 (1, 1) and (1, -1), kept in registers for v_dot2_f32_bf16
  const uint32_t ones = 0x3F803F80u, plus_minus = 0xBF803F80u;
  const float sqrtTBB = __fsqrt_rn(TBB);  // TBB = T B^2 (T B without the rotation)

  // Tile t covers blocks [t BPW, t BPW + BPW); group bw of its lanes takes blocks
  // t BPW + BG bw + b, b < BG.  A block past the last one (ragged last tile) is read as the last
  // block instead and stores nothing, so every load is in bounds and every register holds data.
  constexpr int ES = F32IN ? 4 : 2;  // input element size
  auto tile_in = [&](int64_t t) { return (const char *)xin + t * (BPW * B * ES); };
  auto lane_in = [&](int64_t t) {
    const int64_t last = nb - 1 - t * BPW;  // last block relative to the tile (>= 0)
    const int b0 = BG * bw;
    return (uint32_t)((last < b0 ? (int)last : b0) * B + compress_lane_elems<F32IN>() * j);
  };
  // element step from one run to the next: RS within a block; at BG = 2 the next run is the
  // pair's second block, or the first one again when the second is past the end
  auto run_step = [&](int64_t t) -> uint32_t {
    if constexpr (BG == 1) return RS;
    return (nb - 1 - t * BPW) > BG * bw ? (uint32_t)B : 0u;
  };
  CompressIn<B, F32IN> cur;
  if (wave < ntiles) load_compress_at<B, F32IN>(cur, tile_in(wave), lane_in(wave), run_step(wave));

  for (int64_t tile = wave; tile < ntiles; tile += nwaves) {
    const int64_t blk0 = tile * BPW;  // first block of the tile (wave-uniform)
    CompressIn<B, F32IN> nxt;
    if (LOOP && tile + nwaves < ntiles)
      load_compress_at<B, F32IN>(nxt, tile_in(tile + nwaves), lane_in(tile + nwaves),
                                 run_step(tile + nwaves));

    // Widen, energy and the first butterfly stages.  Blocks past the last one work on a copy
    // of the last block and store nothing.
    float v[N];
    float ss[BG];  // sum(x^2) of each block's values in this lane
    if constexpr (!F32IN) {
      // sums of squares from the packed input: from 32 values per lane and block on (B >= 256)
      // four partial sums, one per dword of a run, added pairwise at the end, so that the
      // rounding error grows with the runs rather than the values (see sum_squares)
      constexpr int KQ = NB >= 32 ? 4 : 1;
      float ssq[BG][KQ];
#pragma unroll
      for (int b = 0; b < BG; ++b)
#pragma unroll
        for (int k = 0; k < KQ; ++k) ssq[b][k] = 0.0f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const u32x4 d = cur.d[g];
        if constexpr (ROT) {
          bf16_butterfly4(d[0], d[1], d[2], d[3], ones, plus_minus, &v[8 * g]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) widen_bf16x2(d[q], v[8 * g + 2 * q], v[8 * g + 2 * q + 1]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          ssq[g * BG / G][q % KQ] = bf16_pair_sumsq(d[q], ssq[g * BG / G][q % KQ]);
      }
#pragma unroll
      for (int b = 0; b < BG; ++b) {
        if constexpr (KQ == 4)
          ss[b] = (ssq[b][0] + ssq[b][1]) + (ssq[b][2] + ssq[b][3]);
        else
          ss[b] = ssq[b][0];
      }
      // register stages within a block: all of them at BG = 1, those inside a run at BG = 2
      if constexpr (ROT) fwht_registers<N, 2, NB>(v);
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[8 * g + q] = __uint_as_float(cur.d[2 * g][q]);
          v[8 * g + 4 + q] = __uint_as_float(cur.d[2 * g + 1][q]);
        }
#pragma unroll
      for (int b = 0; b < BG; ++b) ss[b] = sum_squares<NB>(&v[b * NB]);
      if constexpr (ROT) fwht_registers<N, 1, NB>(v);
    }
    // orthogonal Hadamard rotation, unnormalised: w = H x (1/sqrt(B) and alpha live in s)
    if constexpr (ROT) fwht_lanes<L, N>(v, j);

#pragma unroll
    for (int b = 0; b < BG; ++b) {
      // this block's registers: v[b NB + r], r < NB
      float m = 0.0f;
#pragma unroll
      for (int r = 0; r < NB; ++r) m = fmaxf(m, fabsf(v[b * NB + r]));
      const float M = group_max<L>(m);
      const float SS = group_sum<L>(ss[b]);  // sum(x^2) of the block

      // alpha = sqrt(T B / sum x^2), s = alpha max|w| / (Q sqrt B), codes = code(Q w / max|w|)
      // (Q = 448 for E4M3; without the rotation w = x and s = alpha max|x| / Q).
      // For max|w| in [2^-40, 2^60] every quantity stays normal and sum(x^2) is accurate, so
      // the scales use the single-instruction reciprocal square root (1 ulp, inside the 1e-6
      // bar); the code multiplier Q / max|w| is correctly rounded, so that a quotient that is
      // exactly a rounding midpoint stays exact and rounds to even.
      float cm, alpha, s;
      if (M >= 0x1p-40f && M <= 0x1p60f) {
        const float c = __fdiv_rn(Q, M);
        alpha = fminf(fmaxf(sqrtTB * __builtin_amdgcn_rsqf(SS), 0x1p-126f), 0x1p126f);
        s = alpha * M * invC;
        cm = c * sj;
      } else if (M == 0.0f) {
        // all-zero block: alpha 1, s 0, codes +0
        cm = 0.0f;
        alpha = 1.0f;
        s = 0.0f;
      } else {
        // bfloat16-subnormal or huge block, where sum(x^2) leaves float32's range: the same
        // formulas on the block scaled by the exact power of two 2^k that brings max|w| into
        // [1, 2), with the energy taken from the scaled w (Parseval: sum(w^2) = B sum(x^2)
        // with the rotation, so alpha = sqrt(T B^2 / sum(w^2)) = sqrt(TBB / sum(w^2))), and k
        // taken back out of alpha and s.  The codes do not depend on the scaling.
        const int k = 1 - exponent_of(M);
#pragma unroll
        for (int r = 0; r < NB; ++r) v[b * NB + r] = scale2(v[b * NB + r], k);
        const float Mk = scale2(M, k);
        const float SW = group_sum<L>(sum_squares<NB>(&v[b * NB]));  // 2^2k sum(w^2)
        alpha = fminf(fmaxf(scale2(sqrtTBB * __builtin_amdgcn_rsqf(SW), k), 0x1p-126f),
                      0x1p126f);
        s = scale2(alpha * Mk, -k) * invC;
        cm = __fdiv_rn(Q, Mk) * sj;
      }

      const int64_t blk = blk0 + BG * bw + b;
      if (blk < nb) {
        uint8_t *cb = codes + blk0 * B;  // the tile's codes (wave-uniform)
        if constexpr (!F32IN) {
          const uint32_t co = BG * bw * B + 8 * pj;  // this lane's runs within them
#pragma unroll
          for (int g = b * G / BG; g < (b + 1) * G / BG; ++g) {
            u32x2 w;
            w[0] = encode4<FLAGS>(v[8 * g + 0], v[8 * g + 1], v[8 * g + 2], v[8 * g + 3], cm);
            w[1] = encode4<FLAGS>(v[8 * g + 4], v[8 * g + 5], v[8 * g + 6], v[8 * g + 7], cm);
            st_stream(w, (u32x2 *)(cb + co + RS * g));
          }
        } else {
          // the float32 line layout: this block's runs, through the partner swap
          constexpr int GB = G / BG;  // runs of this block in the lane
          store_codes_line<FLAGS, GB, RS, ROT>(&v[8 * GB * b], cm, pj,
                                               cb + BG * bw * B + RS * GB * b);
        }
        if (j == 0) {
          alpha_out[blk] = alpha;
          scale_out[blk] = s;
        }
      }
    }
    if constexpr (!LOOP) break;
    cur = nxt;
  }
}

// --------------------------------------------------------------------------------------------
// K2: decompress.  x = H (s dec q) / (sqrt(B) alpha), with compress's assignment of each run
// of 64 elements to 8 lanes (bfloat16 output: that of bfloat16 input; float32 output: that of
// float32 input); one tile per
// wavefront, or (LOOP) a grid-stride loop with the next iteration's codes and scales prefetched.

// Decompress keeps 8 lanes per block at every B: its per-block work is small, and at B = 64
// the 8-lane group reads each block's codes, and writes its output, in whole lines.
constexpr int decompress_lanes(int) { return 8; }

// Element layout in a block's 8-lane group.  Each run of 64 elements is spread over the lanes
// and 8 registers per lane; the transform is the same whatever element bits the lane and
// register bits stand for, provided the codes are read and the output written with the same
// assignment (H[i][k] = (-1)^popcount(i & k) does not change when one permutation of the bits
// is applied to both i and k).
//   bfloat16 output: lane j holds elements [8 j, 8 j + 8) of the run (lane bits = element bits
//     3-5), so each lane stores 16 bytes and the group's store instruction writes one whole line.
//   float32 output: lane j holds elements [4 j, 4 j + 4) and [32 + 4 j, 32 + 4 j + 4) (lane
//     bits = element bits 2-4; register bit 2 = element bit 5), so each of the two 16-byte
//     stores of a run covers a whole line across the group.  With the bfloat16 layout each
//     store instruction covered half of every line the group writes: with non-temporal stores
//     that cost a second partial write per line, with plain ones the L2 had to join the halves.
//     The line layout with non-temporal stores was 4-9% faster than the half-line one with plain
//     stores over back-to-back launches through rotating buffers, on 117 M elements at every B
//     (102.0 against 108.2 us at B = 128, 117.1 against 122.6 us at B = 256), with the same
//     output bits.
template <int B, bool F32OUT>
struct DecompressIn {
  u32x2 d[B / (8 * decompress_lanes(B))];  // per run: registers 0-3 and 4-7 as two dwords
  float s, a;
};

template <int B, bool F32OUT>
__device__ __forceinline__ void load_decompress_in(DecompressIn<B, F32OUT> &in,
                                                   const uint8_t *codes, const float *alpha,
                                                   const float *scale, int64_t blk, int j) {
  constexpr int RS = 8 * decompress_lanes(B);
  if constexpr (F32OUT) {
    const uint8_t *cb = codes + blk * B + 4 * j;
#pragma unroll
    for (int g = 0; g < B / RS; ++g) {
      in.d[g][0] = ld_stream((const uint32_t *)(cb + RS * g));
      in.d[g][1] = ld_stream((const uint32_t *)(cb + RS * g + 32));
    }
  } else {
    const uint8_t *cb = codes + blk * B + 8 * j;
#pragma unroll
    for (int g = 0; g < B / RS; ++g) in.d[g] = ld_stream((const u32x2 *)(cb + RS * g));
  }
  in.s = scale[blk];
  in.a = alpha[blk];
}

// LOOP as for k_compress.
template <int B, bool F32OUT, int FLAGS, bool LOOP>
__global__ __launch_bounds__(kThreads) void k_decompress(const uint8_t *__restrict__ codes,
                                                         const float *__restrict__ alpha,
                                                         const float *__restrict__ scale,
                                                         int64_t nb, float inv_sqrt_b,
                                                         void *__restrict__ out) {
  constexpr int L = decompress_lanes(B);
  constexpr int BPW = 64 / L;
  constexpr int RS = 8 * L;
  constexpr int N = B / L;
  constexpr int G = N / 8;
  constexpr bool ROT = !(FLAGS & kNoRotation);
  const int lane = threadIdx.x & 63;
  const int j = lane & (L - 1);
  const int bw = lane / L;
  const int pj = ROT ? lane_perm<L>(j) : j;
  const float sj = ROT ? lane_sign<L>(j) : 1.0f;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t ntiles = (int64_t)(((uint64_t)nb + BPW - 1) / BPW);  // nb >= 0

  DecompressIn<B, F32OUT> cur;  // groups past the last block re-read the last block, store nothing
  if (wave < ntiles)
    load_decompress_in<B, F32OUT>(cur, codes, alpha, scale, min(wave * BPW + bw, nb - 1), j);

  for (int64_t tile = wave; tile < ntiles; tile += nwaves) {
    const int64_t blk = tile * BPW + bw;
    const bool active = blk < nb;
    DecompressIn<B, F32OUT> nxt;
    if (LOOP && tile + nwaves < ntiles)
      load_decompress_in<B, F32OUT>(nxt, codes, alpha, scale,
                                    min((tile + nwaves) * BPW + bw, nb - 1), j);

    float v[N];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint32_t w0 = cur.d[g][0], w1 = cur.d[g][1];
      decode4<FLAGS>(w0, v[8 * g + 0], v[8 * g + 1], v[8 * g + 2], v[8 * g + 3]);
      decode4<FLAGS>(w1, v[8 * g + 4], v[8 * g + 5], v[8 * g + 6], v[8 * g + 7]);
    }
    const float s = cur.s, a = cur.a;

    // The decoded values are multiples of 2^-9 below 2^8.81 (E4M3) or integers below 2^7
    // (INT8), so every partial sum of the transform is exact in float32 until it passes 2^15
    // (E4M3) or 2^24 (INT8: never).  The first six stages stay below 2^15 (64 * 448 < 2^15), so
    // for B <= 128 only the last stage can round, once, relative to the output itself.  At
    // B >= 256 (E4M3) a rounding in a later stage but the last would be relative to a partial
    // sum that the remaining stages may cancel, so the per-element error would be unbounded: the
    // six exact stages run first (within each run of 8 registers, then across the lanes), and
    // the remaining R stages run in float64 (exact there), rounded once at the end.  The
    // transform's output is then correctly rounded at every B.  (Taking the float64 stages only
    // for blocks whose partial sums could pass 2^15 cost registers and was slower; int32
    // stages on the values in units of 2^-9, exact as well and bit for bit the same, were
    // 0.5-3.5% slower.)
    if constexpr (ROT) {
      if constexpr (N <= 16 || (FLAGS & kInt8)) {
        fwht_registers<N, 1>(v);
        fwht_lanes<L, N>(v, j);
      } else {
        fwht_registers<N, 1, 8>(v);
        fwht_lanes<L, N>(v, j);
        // The remaining R = log2(N / 8) stages only combine registers with the same index mod 8:
        // one such class of K = N / 8 registers at a time, in float64, where every partial sum
        // (a multiple of 2^-9 below 2^(15 + R)) is exact; the conversion back is the one rounding.
        constexpr int K = N / 8;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          double d[K];
#pragma unroll
          for (int k = 0; k < K; ++k) d[k] = (double)v[c + 8 * k];
#pragma unroll
          for (int h = 1; h < K; h <<= 1)
#pragma unroll
            for (int i = 0; i < K; i += 2 * h)
#pragma unroll
              for (int k = i; k < i + h; ++k) {
                const double x = d[k], y = d[k + h];
                d[k] = x + y;
                d[k + h] = x - y;
              }
#pragma unroll
          for (int k = 0; k < K; ++k) v[c + 8 * k] = (float)d[k];
        }
      }
    }

    // (v * s / sqrt(B)) / alpha as two products: s / (sqrt(B) alpha) alone can fall below the
    // normal range when alpha is large, the two-step form only rounds the final value there.
    const float f = (s == 0.0f) ? 0.0f : sj * (s * inv_sqrt_b);
    const float ra = __frcp_rn(a);

    if (active) {
      if constexpr (F32OUT) {
        // the line layout above: registers 0-3 of a run at 4 pj, registers 4-7 at 32 + 4 pj
        float *ob = (float *)out + blk * B + 4 * pj;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          u32x4 w0, w1;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            w0[q] = __float_as_uint(fmaf(v[8 * g + q], f, 0.0f) * ra);
            w1[q] = __float_as_uint(fmaf(v[8 * g + 4 + q], f, 0.0f) * ra);
          }
          st_stream(w0, (u32x4 *)(ob + RS * g));
          st_stream(w1, (u32x4 *)(ob + RS * g + 32));
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
          st_stream(w, (u32x4 *)(ob + RS * g));
        }
      }
    }
    if constexpr (!LOOP) break;
    cur = nxt;
  }
}

// --------------------------------------------------------------------------------------------
// K3: reduce.  B/16 lanes per block, 16 consecutive codes per lane (one 16-byte load per
// contribution), no Hadamard.  PB > 0: exactly PB contributions, all loads issued before any
// arithmetic; PB = 0: any P, in chunks of 8.  Contribution p's codes start at codes + p cstride
// and its scales at alpha + p astride, scale + p sstride (cstride = n, astride = sstride = nb
// for contiguous stacks).  (8 codes per lane, which halves the registers and allows eight
// wavefronts per SIMD instead of five, measured 2-11% slower.)

template <int B, int PB, int FLAGS>
__global__ __launch_bounds__(kThreads) void k_reduce(const uint8_t *__restrict__ codes,
                                                     const float *__restrict__ alpha,
                                                     const float *__restrict__ scale, int P,
                                                     int64_t cstride, int64_t astride,
                                                     int64_t sstride, int64_t nb, float TB,
                                                     uint8_t *__restrict__ codes_out,
                                                     float *__restrict__ alpha_out,
                                                     float *__restrict__ scale_out) {
  constexpr int L = B / 16;    // lanes per block
  constexpr int BPW = 64 / L;  // blocks per wavefront
  constexpr int CH = PB > 0 ? PB : 8;  // contributions loaded together
  // low bits of g cleared so that g times a code value is exact in float64: E4M3 values have
  // at most 4 significant bits (g keeps 49), INT8 values at most 7 (g keeps 46)
  constexpr long long kGMask = (FLAGS & kInt8) ? ~0x7FLL : ~0xFLL;
  if constexpr (PB > 0) P = PB;
  const int lane = threadIdx.x & 63;
  const int j = lane % L;
  const int bw = lane / L;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t ntiles = (int64_t)(((uint64_t)nb + BPW - 1) / BPW);  // nb >= 0

  for (int64_t tile = wave; tile < ntiles; tile += nwaves) {
    const int64_t blk = tile * BPW + bw;
    const bool active = blk < nb;
    const int64_t cblk = active ? blk : nb - 1;  // groups past the end re-read the last block
    const uint8_t *cb = codes + cblk * B + 16 * j;

    // r = sum_p g_p dec(q_p) with g_p = s_p / alpha_p, accumulated in float64.  g_p is cut to
    // 49 significant bits (46 for INT8 codes; a relative change below 2^-45), so that its
    // product with a code value is exact in float64; the only roundings are those of
    // the running sum, each within 2^-53 of it.  Each element of r is therefore within
    // 2^-44 of the sum of its terms' magnitudes: contributions that cancel down to about 2^-25
    // of their peaks still requantise like the exact sum, and a contribution and its exact
    // negation cancel to exactly zero when no smaller term is summed between them (one added
    // to the larger first is rounded away with it, as in any float64 sum).  A zero block
    // (s_p = 0) contributes exact zeros.
    double r64[16];
    for (int p0 = 0; p0 < P; p0 += CH) {
      u32x4 d[CH];
      float sp[CH], ap[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (PB > 0 || p0 + c < P) {
          d[c] = ld_stream((const u32x4 *)(cb + (int64_t)(p0 + c) * cstride));
          sp[c] = scale[(int64_t)(p0 + c) * sstride + cblk];
          ap[c] = alpha[(int64_t)(p0 + c) * astride + cblk];
        }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        if (PB > 0 || p0 + c < P) {
          // 1/alpha in float64: hardware reciprocal refined by two Newton steps
          const double ad = (double)ap[c];
          double ri = __builtin_amdgcn_rcp(ad);
          ri = fma(ri, fma(-ad, ri, 1.0), ri);
          ri = fma(ri, fma(-ad, ri, 1.0), ri);
          const double g = __longlong_as_double(__double_as_longlong((double)sp[c] * ri) & kGMask);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float a0, a1, a2, a3;
            decode4<FLAGS>(d[c][q], a0, a1, a2, a3);
            if (p0 + c == 0) {
              r64[4 * q + 0] = (double)a0 * g;
              r64[4 * q + 1] = (double)a1 * g;
              r64[4 * q + 2] = (double)a2 * g;
              r64[4 * q + 3] = (double)a3 * g;
            } else {
              r64[4 * q + 0] = fma((double)a0, g, r64[4 * q + 0]);
              r64[4 * q + 1] = fma((double)a1, g, r64[4 * q + 1]);
              r64[4 * q + 2] = fma((double)a2, g, r64[4 * q + 2]);
              r64[4 * q + 3] = fma((double)a3, g, r64[4 * q + 3]);
            }
          }
        }
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
    int E = 0;
    if (M != 0.0f && !(M >= 0x1p-100f && M <= 0x1p100f)) {
      // Tiny or huge sum (bfloat16-subnormal blocks, or contributions that cancelled):
      // rescale the float64 sum so that its largest magnitude lies in [1, 2) before rounding
      // it to float32.
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
    float cm, a_out, s_out;
    constexpr float Q = qmax_of<FLAGS>();
    scales_exact<L, 16>(r, M, E, TB, Q, Q, 1.0f, cm, a_out, s_out);
    if (active) {
      u32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = encode4<FLAGS>(r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3], cm);
      st_stream(w, (u32x4 *)(codes_out + blk * B + 16 * j));
      if (j == 0) {
        alpha_out[blk] = a_out;
        scale_out[blk] = s_out;
      }
    }
  }
}

// --------------------------------------------------------------------------------------------
// K4: local gradient accumulation.  The compressed main gradient (codes, alpha, s) plus a dense
// local gradient g, requantised.  In the rotated domain the main gradient needs no transform:
// H xhat = sqrt(B) (s / alpha) dec(q) (H unnormalised, (H / sqrt(B))^2 = I), so
//   w = H z = H g + sqrt(B) (s / alpha) dec(q),
// and w is requantised exactly like compress requantises H x.  Lane layout: compress's
// assignment of elements to lanes for the gradient's type (runs of 8 per lane for bfloat16, with
// 4 lanes per block at B = 64; the whole-line layout for float32 at B >= 128, with the partner
// swap for the code stores; runs of 8 for float32 at B = 64, whose 4-lane runs are one line).
// Each lane reads the main gradient's codes at the positions its results take, so the call may
// work in place: every code a group stores depends, through the group's maximum, on all of the
// group's loaded codes.  The line layout made the float32-gradient accumulation 6-8% faster over
// rotating buffers (117 M elements: 117.5 against 124.3 us at B = 128, 120.8 against 131.0 us
// at B = 512).
//
// Two launches.  k_accumulate works in float32: its rounding errors are ~2^-24 of the larger
// of the two terms (the float32 transform of g, the product with the factor), which keeps the
// energy and the codes' values to the accuracy of compress as long as the terms do not cancel.
// Where they do (the sum's peak under half the larger term's: about 1e-4 of the blocks of
// independent gradients, but 15% of blocks that share outlier channels of random sign) it sets
// the block aside: it writes only alpha_out = -alpha (alpha is otherwise positive), so the
// block's inputs stay intact even in place.  k_accumulate_fix finds those blocks and redoes them
// with an exact split of the transform (below).  Keeping that code out of the streaming kernel
// keeps the streaming kernel's registers, and so its occupancy, at those of compress.

template <int B, bool F32IN, int FLAGS>
__global__ __launch_bounds__(kThreads) void k_accumulate(
    const uint8_t *codes, const float *alpha, const float *scale, const void *__restrict__ grad,
    int64_t nb, float TBB, float sqrtTBB, float gscale, float C, float invC, uint8_t *codes_out,
    float *alpha_out, float *scale_out) {
  constexpr int L = lanes_per_block(B);
  constexpr int BPW = 64 / L;
  constexpr int RS = 8 * L;
  constexpr int N = B / L;
  constexpr int G = N / 8;
  constexpr bool ROT = !(FLAGS & kNoRotation);
  constexpr float Q = qmax_of<FLAGS>();
  const int lane = threadIdx.x & 63;
  const int j = lane & (L - 1);
  const int bw = lane / L;
  const int pj = ROT ? lane_perm<L>(j) : j;
  const float sj = ROT ? lane_sign<L>(j) : 1.0f;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t ntiles = (int64_t)(((uint64_t)nb + BPW - 1) / BPW);  // nb >= 0
  const uint32_t ones = 0x3F803F80u, plus_minus = 0xBF803F80u;

  // float32 gradient at 8 lanes per block: lane j holds elements [4 j, 4 j + 4) and
  // [32 + 4 j, 32 + 4 j + 4) of each run (register bit 2 = element bit 5), as in compress
  constexpr bool LINE = F32IN && L == 8;
  for (int64_t tile = wave; tile < ntiles; tile += nwaves) {
    const int64_t blk = tile * BPW + bw;
    const bool active = blk < nb;
    const int64_t cblk = active ? blk : nb - 1;  // groups past the end re-read the last block
    CompressIn<B, F32IN> in;
    u32x2 qd[G];  // the main gradient's codes at this lane's result positions
    if constexpr (LINE) {
      const float *xb = (const float *)grad + cblk * B + 4 * j;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        in.d[2 * g] = ld_stream((const u32x4 *)(xb + RS * g));
        in.d[2 * g + 1] = ld_stream((const u32x4 *)(xb + RS * g + 32));
      }
      const uint8_t *cq = codes + cblk * B + 4 * pj;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        qd[g][0] = *(const uint32_t *)(cq + RS * g);
        qd[g][1] = *(const uint32_t *)(cq + RS * g + 32);
      }
    } else {
      load_compress_in<B, F32IN>(in, grad, cblk, j);
#pragma unroll
      for (int g = 0; g < G; ++g) qd[g] = *(const u32x2 *)(codes + cblk * B + RS * g + 8 * pj);
    }
    const float sp = scale[cblk], ap = alpha[cblk];

    float v[N];
    if constexpr (!F32IN) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const u32x4 d = in.d[g];
        if constexpr (ROT) {
          bf16_butterfly4(d[0], d[1], d[2], d[3], ones, plus_minus, &v[8 * g]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) widen_bf16x2(d[q], v[8 * g + 2 * q], v[8 * g + 2 * q + 1]);
        }
      }
      if constexpr (ROT) fwht_registers<N, 2>(v);
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[8 * g + q] = __uint_as_float(in.d[2 * g][q]);
          v[8 * g + 4 + q] = __uint_as_float(in.d[2 * g + 1][q]);
        }
      if constexpr (ROT) fwht_registers<N, 1>(v);
    }
    // lane j: sj * (H g) at positions RS g + 8 pj + e (line layout: RS g + 4 pj + e and
    // RS g + 32 + 4 pj + e, e < 4)
    if constexpr (ROT) fwht_lanes<L, N>(v, j);

    float mh = 0.0f;  // largest |H g| of the block
#pragma unroll
    for (int r = 0; r < N; ++r) mh = fmaxf(mh, fabsf(v[r]));
    mh = group_max<L>(mh);

    // Add the main gradient in the same (signed, permuted) positions, with factor
    // gscale * s / alpha.  Where s / alpha leaves float32's range (alpha clamped at 2^126 on a
    // bfloat16-subnormal main block) both terms are carried as v * 2^E0, E0 the larger of their
    // exponents (|gscale (s / alpha) dec| < 2^(es - ea + 15)), with the factor's mantissa and
    // exponent apart.
    // A main term below 2^-60 of the block's largest |H g| cannot move alpha by more than 2^-60
    // relative, nor a code unless its quotient lies within 2^-51 of a rounding midpoint: it is
    // left out rather than carried through that path (mh >= 2^(exponent_of(mh) - 1)).
    const int es = exponent_of(sp), ea = exponent_of(ap);
    const bool negligible = mh != 0.0f && es - ea + 15 <= exponent_of(mh) - 61;
    const bool in_range = (sp == 0.0f) || negligible || (es - ea > -100 && es - ea < 100);
    float gm;
    int E0 = 0;
    if (in_range) {
      // the factor needs no correct rounding: the codes are decided against the sum's own
      // maximum, and a 1-ulp change of it moves w by 2^-23 of the main term
      gm = (sp == 0.0f || negligible)
               ? 0.0f
               : sj * (gscale * (sp * __builtin_amdgcn_rcpf(ap)));
    } else {
      E0 = max(mh == 0.0f ? -(1 << 20) : exponent_of(mh), es - ea + 15);
#pragma unroll
      for (int r = 0; r < N; ++r) v[r] = scale2(v[r], -E0);
      mh = scale2(mh, -E0);
      gm = sj * scale2(gscale * __fdiv_rn(mantissa_of(sp), mantissa_of(ap)), es - ea - E0);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d[8];
      decode4<FLAGS>(qd[g][0], d[0], d[1], d[2], d[3]);
      decode4<FLAGS>(qd[g][1], d[4], d[5], d[6], d[7]);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[8 * g + e] = fmaf(d[e], gm, v[8 * g + e]);
    }

    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < N; ++r) m = fmaxf(m, fabsf(v[r]));
    const float M = group_max<L>(m);

    // float32 keeps w to ~2^-24 of the larger term; where the terms cancel that is too coarse
    // (see above), and the block is left to k_accumulate_fix
    const bool defer = M < 0.5f * fmaxf(mh, fabsf(gm) * Q);
    float cm = 0.0f, a_out = 1.0f, s_out = 0.0f;
    if (!defer) {
      if (E0 == 0 && M >= 0x1p-40f && M <= 0x1p56f) {
        // energy of z from w (Parseval): alpha = sqrt(T B^2 / sum w^2); with M in this range
        // the sum of squares stays within float32 (at most B M^2 <= 2^121), and squares that
        // underflow are below 2^-70 of the largest
        const float SW = group_sum<L>(sum_squares<N>(v));
        const float c = __fdiv_rn(Q, M);
        a_out = fminf(fmaxf(sqrtTBB * __builtin_amdgcn_rsqf(SW), 0x1p-126f), 0x1p126f);
        s_out = a_out * M * invC;
        cm = c * sj;
      } else {
        scales_exact<L, N>(v, M, E0, TBB, Q, C, sj, cm, a_out, s_out);
      }
    }

    if (active) {
      if (!defer) {
        if constexpr (LINE) {
          store_codes_line<FLAGS, G, RS, ROT>(v, cm, pj, codes_out + blk * B);
        } else {
          uint8_t *cb = codes_out + blk * B + 8 * pj;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            u32x2 w;
            w[0] = encode4<FLAGS>(v[8 * g + 0], v[8 * g + 1], v[8 * g + 2], v[8 * g + 3], cm);
            w[1] = encode4<FLAGS>(v[8 * g + 4], v[8 * g + 5], v[8 * g + 6], v[8 * g + 7], cm);
            st_stream(w, (u32x2 *)(cb + RS * g));
          }
        }
        if (j == 0) {
          alpha_out[blk] = a_out;
          scale_out[blk] = s_out;
        }
      } else if (j == 0) {
        alpha_out[blk] = -ap;
      }
    }
  }
}

// The inputs of one set-aside block, as lane j of its group reads them.
template <int B, bool F32IN>
struct FixIn {
  CompressIn<B, F32IN> in;                  // the local gradient g
  u32x2 qd[B / lanes_per_block(B) / 8];     // the main gradient's codes
  float sp, ap;                             // its s and alpha
};

template <int B, bool F32IN, int FLAGS>
__device__ __forceinline__ void load_fix_in(FixIn<B, F32IN> &f, const uint8_t *codes,
                                            const float *scale, const void *__restrict__ grad,
                                            const float *alpha_out, int64_t blk, int j) {
  constexpr int L = lanes_per_block(B);
  constexpr int RS = 8 * L;
  constexpr int G = B / L / 8;
  constexpr bool ROT = !(FLAGS & kNoRotation);
  load_compress_in<B, F32IN>(f.in, grad, blk, j);
  // The lane network sends lane j's result to position pj.  Reading lane j's codes from 8 qj
  // instead of 8 j, with qj = j ^ (3 bit2(j)) at L = 8 (the transpose of that GF(2)-linear
  // permutation; identity at L = 4 and without the rotation), makes the network's output land
  // at lane j's own positions, those of g, with the sign sj (enumerated on the unit vectors).
  const int qj = ROT && L == 8 ? j ^ (((j >> 2) & 1) * 3) : j;
#pragma unroll
  for (int g = 0; g < G; ++g) f.qd[g] = *(const u32x2 *)(codes + blk * B + RS * g + 8 * qj);
  f.sp = scale[blk];
  f.ap = -alpha_out[blk];
}

// One set-aside block, by the group of L lanes j = 0..L-1 that holds it (runs of 8 consecutive
// elements per lane for either gradient type).  Its codes and s are still those of the main gradient (never written) and
// alpha_out holds -alpha.  `active` = 0: work on the block but store nothing.  Lane j reads codes
// at positions 8 qj and writes them at 8 pj, where another lane of the group read; in place that
// is safe because every stored value depends, through the lane exchanges, on all of the group's
// loaded codes, so the group's loads have completed before any of its stores.
//
// The sum is formed with the roundings of the plain definition, so that it is exact wherever
// the terms cancel exactly.  The transform of the decoded codes is exact: the first stages in
// float32 (3 within each run of 8 registers, log2(L) across the lanes: partial sums of multiples
// of 2^-9 below 64 * 448 < 2^15), the remaining ones in float64.  Multiplying it by s is exact
// too (24 + 27 significant bits), the divisions by sqrt(B) and by alpha round once each, and
// adding g rounds once: z matches the float64 reconstruction plus g bit for bit.  Everything
// after z errs relative to z itself.  z is rotated as compress rotates its input: scaled by
// 2^(K - E) with max|z| < 2^E and split into integers r = rint(t) and remainders l = t - r in
// [-1/2, 1/2].  |r| <= 2^K with K = 24 - log2(B), so every partial sum of H r is an integer of
// at most 2^24 and the transform of r is exact; the transform of l errs by ~2^-18 of 2^K at most.
template <int B, bool F32IN, int FLAGS>
__device__ __forceinline__ void accumulate_block_split(
    const FixIn<B, F32IN> &f, int64_t blk, bool active, int j, float TBB, float C, double root_b,
    uint8_t *codes_out, float *alpha_out, float *scale_out) {
  constexpr int L = lanes_per_block(B);
  constexpr int RS = 8 * L;
  constexpr int N = B / L;
  constexpr int G = N / 8;
  constexpr int NC = N / 8;  // registers per class of the float64 stages
  constexpr bool ROT = !(FLAGS & kNoRotation);
  constexpr float Q = qmax_of<FLAGS>();
  constexpr int K = 24 - (B == 64 ? 6 : B == 128 ? 7 : B == 256 ? 8 : 9);
  const int pj = ROT ? lane_perm<L>(j) : j;
  const float sj = ROT ? lane_sign<L>(j) : 1.0f;
  const CompressIn<B, F32IN> &in = f.in;
  const u32x2 *qd = f.qd;
  const float sp = f.sp, ap = f.ap;

  float gv[N];  // g at positions RS g + 8 j + e
  if constexpr (!F32IN) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        widen_bf16x2(in.d[g][q], gv[8 * g + 2 * q], gv[8 * g + 2 * q + 1]);
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        gv[8 * g + q] = __uint_as_float(in.d[2 * g][q]);
        gv[8 * g + 4 + q] = __uint_as_float(in.d[2 * g + 1][q]);
      }
  }
  float v[N];  // decoded codes at positions RS g + 8 qj + e; after the transform lane j holds
               // sj * (H dec) at positions RS g + 8 j + e, those of g
#pragma unroll
  for (int g = 0; g < G; ++g) {
    decode4<FLAGS>(qd[g][0], v[8 * g + 0], v[8 * g + 1], v[8 * g + 2], v[8 * g + 3]);
    decode4<FLAGS>(qd[g][1], v[8 * g + 4], v[8 * g + 5], v[8 * g + 6], v[8 * g + 7]);
  }
  if constexpr (ROT) {
    fwht_registers<N, 1, 8>(v);
    fwht_lanes<L, N>(v, j);
  }
  double z[N];
#pragma unroll
  for (int i = 0; i < N; ++i) z[i] = (double)v[i];
  if constexpr (ROT && NC > 1) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int h = 1; h < NC; h <<= 1)
#pragma unroll
        for (int i = 0; i < NC; i += 2 * h)
#pragma unroll
          for (int k = i; k < i + h; ++k) {
            const double x = z[c + 8 * k], y = z[c + 8 * (k + h)];
            z[c + 8 * k] = x + y;
            z[c + 8 * (k + h)] = x - y;
          }
  }
  const double sd = (double)sj * (double)sp;  // sj = +-1: exact
  // m / b rounded to nearest from y = RN(1 / b): q = RN(m y) is within an ulp of m / b, the FMA
  // gives its residual m - b q exactly, and q + (m - b q) y rounds to RN(m / b) (Markstein's
  // theorem); one division per block instead of one per element
  const auto div_rn = [](double m, double b, double y) {
    const double q = m * y;
    return fma(fma(-q, b, m), y, q);
  };
  const double ya = 1.0 / (double)ap, yb = 1.0 / root_b;
  int ez = 0;  // biased float64 exponent of max|z|; 0 only if every z is zero
#pragma unroll
  for (int i = 0; i < N; ++i) {
    double m = sd * z[i];  // exact
    if constexpr (ROT) {
      if constexpr (B == 64 || B == 256) m = m * (B == 64 ? 0.125 : 0.0625);  // exact
      else m = div_rn(m, root_b, yb);
    }
    m = div_rn(m, (double)ap, ya);
    z[i] = (sp == 0.0f ? 0.0 : m) + (double)gv[i];
    ez = max(ez, (int)((__double_as_longlong(z[i]) >> 52) & 0x7ff));
  }
  ez = group_max_i<L>(ez);
  // sums of float32 values are float64 normals or zero, so max|z| < 2^E with E = ez - 1022
  const int E = ez == 0 ? 0 : ez - 1022;
  float r[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const double t = __builtin_amdgcn_ldexp(z[i], K - E);
    if constexpr (ROT) {
      const double ri = __builtin_rint(t);
      r[i] = (float)ri;
      v[i] = (float)(t - ri);  // the remainder l
    } else {
      r[i] = (float)t;  // one rounding, relative to z
    }
  }
  if constexpr (ROT) {
    fwht_registers<N, 1>(r);
    fwht_lanes<L, N>(r, j);  // lane j: sj * (H r) at positions RS g + 8 pj + e
    fwht_registers<N, 1>(v);
    fwht_lanes<L, N>(v, j);
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = r[i] + v[i];
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) m = fmaxf(m, fabsf(r[i]));
  const float M = group_max<L>(m);
  float cm, a_out, s_out;
  scales_exact<L, N>(r, M, E - K, TBB, Q, C, sj, cm, a_out, s_out);
  if (active) {
    uint8_t *cb = codes_out + blk * B + 8 * pj;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      u32x2 q;
      q[0] = encode4<FLAGS>(r[8 * g + 0], r[8 * g + 1], r[8 * g + 2], r[8 * g + 3], cm);
      q[1] = encode4<FLAGS>(r[8 * g + 4], r[8 * g + 5], r[8 * g + 6], r[8 * g + 7], cm);
      *(u32x2 *)(cb + RS * g) = q;
    }
    if (j == 0) {
      alpha_out[blk] = a_out;
      scale_out[blk] = s_out;
    }
  }
}

// Runs of 64 blocks that one wavefront of k_accumulate_fix scans.  Deeper scans (4, 8, 16 runs)
// measured 1-8% slower with almost nothing to redo (GPT-13B-shaped gradients) and 4-34% slower
// with 15% of the blocks to redo (Qwen-shaped shards that share outlier channels): fewer
// wavefronts then carry the redone blocks.  One run per wavefront was about 1% slower in both.
constexpr int kFixRuns = 2;

// Position of the n-th set bit (n counted from 0) of m, which has more than n set bits: a binary
// search on the population counts of the low halves.
__device__ __forceinline__ int nth_set_bit(uint64_t m, int n) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const int c = __popcll(m & ((1ull << w) - 1));
    if (n >= c) {
      n -= c;
      m >>= w;
      pos += w;
    }
  }
  return pos;
}

// Finds the blocks k_accumulate set aside (alpha_out < 0) and redoes them.  A wavefront reads the
// alphas of kRuns x 64 consecutive blocks at once (kRuns loads in flight per lane) and deals the
// marked blocks of all its runs out in rounds of 64 / L, one block per group of L lanes, with the
// next round's inputs loaded before the current round's arithmetic.  Groups left without a block
// in the last round redo that round's first block and store nothing; a round's loads never touch
// a block that an earlier round stores (each marked block is in exactly one round), so working
// in place is safe across rounds as within one.
template <int B, bool F32IN, int FLAGS>
__global__ __launch_bounds__(kThreads) void k_accumulate_fix(
    const uint8_t *codes, const float *scale, const void *__restrict__ grad, int64_t nb,
    float TBB, float C, double root_b, uint8_t *codes_out, float *alpha_out, float *scale_out) {
  constexpr int kRuns = kFixRuns;
  constexpr int L = lanes_per_block(B);
  constexpr int BPW = 64 / L;  // blocks worked on at once: one per group of L lanes
  const int lane = threadIdx.x & 63;
  const int j = lane & (L - 1);
  const int bw = lane / L;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t nscan = (nb + 64 * kRuns - 1) / (64 * kRuns);

  for (int64_t t = wave; t < nscan; t += nwaves) {
    float am[kRuns];
#pragma unroll
    for (int run = 0; run < kRuns; ++run) {
      const int64_t b = (t * kRuns + run) * 64 + lane;
      am[run] = b < nb ? alpha_out[b] : 1.0f;
    }
    uint64_t mask[kRuns];
    int count = 0;  // marked blocks of the scan (wave-uniform)
#pragma unroll
    for (int run = 0; run < kRuns; ++run) {
      mask[run] = __ballot(am[run] < 0.0f);
      count += __popcll(mask[run]);
    }
    // the idx-th marked block of the scan (idx < count), as an offset from its first block
    const auto marked = [&](int idx) {
      int off = 0;
#pragma unroll
      for (int run = kRuns - 1; run >= 0; --run) {
        int before = 0;  // marked blocks in the runs before this one
#pragma unroll
        for (int r = 0; r < run; ++r) before += __popcll(mask[r]);
        if (idx >= before && idx < before + __popcll(mask[run]))
          off = run * 64 + nth_set_bit(mask[run], idx - before);
      }
      return off;
    };
    const int rounds = (count + BPW - 1) / BPW;
    if (rounds == 0) continue;
    const int64_t base = t * kRuns * 64;  // the scan's first block (wave-uniform)
    // group bw's block of round r: the (r BPW + bw)-th marked one, or the round's first
    const auto block_of = [&](int r) {
      const int idx = r * BPW + bw;
      return marked(idx < count ? idx : r * BPW);
    };
    FixIn<B, F32IN> cur;
    load_fix_in<B, F32IN, FLAGS>(cur, codes, scale, grad, alpha_out, base + block_of(0), j);
    for (int r = 0; r < rounds; ++r) {
      FixIn<B, F32IN> nxt;
      if (r + 1 < rounds)
        load_fix_in<B, F32IN, FLAGS>(nxt, codes, scale, grad, alpha_out, base + block_of(r + 1), j);
      // the block is located again rather than carried over: that keeps the registers at five
      // wavefronts per SIMD
      accumulate_block_split<B, F32IN, FLAGS>(cur, base + block_of(r), r * BPW + bw < count, j,
                                              TBB, C, root_b, codes_out, alpha_out, scale_out);
      cur = nxt;
    }
  }
}

}  // namespace tfp8

// ============================================================================================
// Host side of the C ABI: argument checks (before any HIP call), kernel choice, launch shape.

// Build-time caps on each kernel's grid, in workgroups per compute unit (0 = no cap: one
// wavefront per tile, up to 2^30 work-items).  The library is built without them.  A build with
// them set makes the kernels' grid-stride loops run at small sizes, for tests of those loops;
// the caps change only the grid the host picks, not the kernels.
#ifndef TFP8_COMPRESS_WGS_PER_CU
#define TFP8_COMPRESS_WGS_PER_CU 0
#endif
#ifndef TFP8_DECOMPRESS_WGS_PER_CU
#define TFP8_DECOMPRESS_WGS_PER_CU 0
#endif
#ifndef TFP8_REDUCE_WGS_PER_CU
#define TFP8_REDUCE_WGS_PER_CU 0
#endif
#ifndef TFP8_ACCUMULATE_FIX_WGS_PER_CU
#define TFP8_ACCUMULATE_FIX_WGS_PER_CU 0
#endif

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

// Workgroups for a launch with one wavefront per tile, capped at `per_cu` workgroups per
// compute unit (0: no cap) beyond which the wavefronts loop over tiles.  Measured on MI355X:
// compress, decompress and the reduce all stream fastest with one tile per wavefront and no loop
// (the hardware keeps the CUs fed as wavefronts retire).  With the caches flushed before each
// launch, caps of 2-32 workgroups per CU with prefetching loops were 1-16% slower on
// 34-940 M-element inputs; over back-to-back launches through rotating buffers the uncapped
// reduce was 4% faster than at 32 workgroups per CU on the full Qwen-shaped tensor, and equal
// at one rank's share.
int cu_count() {
  // compute units of the current device, looked up once per device (any thread may race to
  // fill an entry; they all store the same value)
  constexpr int kMaxDevices = 64;
  static std::atomic<int> by_device[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int cus = by_device[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    by_device[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// Compress of a large input is 2-4% faster with 64-thread workgroups and each XCD on a
// contiguous eighth of the tiles: 77% -> 80% of HBM peak for every bf16 input measured from
// 1.9 to 4.3 GB.  At 1.1 GB the two shapes tie, and on inputs of 134-268 MB the remapped one is
// 3-10% slower, hence the threshold.  At B = 64, whose lane groups now read whole lines as at
// B = 128, the remapped shape is 1% faster on 1.9 GB.  Decompress and the reduce were slower
// remapped.
constexpr int64_t kCompressRemapMinBytes = (int64_t)3 << 29;  // 1.5 GiB of input

// The cap without `per_cu` keeps gridDim.x * nt (the work-items of the launch, a 32-bit count
// in the dispatch packet) at 2^30; larger inputs loop.  Under the XCD remap the count is
// rounded up to a multiple of 8, and the extra wavefronts find no tile.
unsigned grid_for(int64_t tiles, int per_cu, int nt = kThreads, bool remap = false) {
  const int64_t wgs = (tiles + (nt / 64) - 1) / (nt / 64);
  const int64_t cap = per_cu > 0 ? (int64_t)cu_count() * per_cu : ((int64_t)1 << 30) / nt;
  int64_t g = wgs < cap ? (wgs > 0 ? wgs : 1) : cap;
  if (remap) g = (g + 7) / 8 * 8;
  return (unsigned)g;
}

// Launches `kernel` with `args` converted to its parameter types, and returns the status of this
// launch itself (hipLaunchKernel reports it directly, so an error left over from an earlier,
// unrelated HIP call is not taken for this launch's).
template <typename... KArgs, typename... Args>
tfp8_status launch(void (*kernel)(KArgs...), unsigned grid, int threads, hipStream_t st,
                   Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> held(static_cast<KArgs>(args)...);
  void *argv[sizeof...(KArgs)];
  std::apply([&argv](auto &...a) {
    int i = 0;
    ((argv[i++] = (void *)&a), ...);
  }, held);
  return hipLaunchKernel((const void *)kernel, dim3(grid), dim3(threads), argv, 0, st) ==
                 hipSuccess
             ? TFP8_OK
             : TFP8_E_HIP;
}

template <int B, bool F32, int FLAGS>
tfp8_status launch_compress_t(const void *x, int64_t nb, float target, uint8_t *codes,
                              float *alpha, float *scale, hipStream_t st) {
  constexpr bool ROT = !(FLAGS & kNoRotation);
  const double Q = qmax_of<FLAGS>();
  // energy of v: sum(v^2) = B sum(x^2) with the (unnormalised) rotation, sum(x^2) without
  const float TBB = target * (float)B * (ROT ? (float)B : 1.0f);  // exact: powers of two
  const float sqrtTB = (float)sqrt((double)target * B);
  const double Cd = ROT ? Q * sqrt((double)B) : Q;
  const float C = (float)Cd, invC = (float)(1.0 / Cd);
  constexpr int BPW = 64 / 8 * compress_blocks_per_group(B);  // blocks per tile
  // Large inputs stream faster with one wavefront per workgroup and each XCD on a contiguous
  // eighth of the tiles; smaller ones with 4 wavefronts per workgroup in dispatch order.
  const bool remap = nb * B * (F32 ? 4 : 2) >= kCompressRemapMinBytes;
  const int nt = remap ? 64 : kThreads;
  const int64_t tiles = (nb + BPW - 1) / BPW;
  const unsigned grid = grid_for(tiles, TFP8_COMPRESS_WGS_PER_CU, nt, remap);
  if ((int64_t)grid * (nt / 64) < tiles)  // capped launch: wavefronts loop over tiles
    return launch(k_compress<B, F32, FLAGS, true>, grid, nt, st, x, nb, TBB, sqrtTB, C, invC,
                  codes, alpha, scale, nt / 64, remap);
  return launch(k_compress<B, F32, FLAGS, false>, grid, nt, st, x, nb, TBB, sqrtTB, C, invC,
                codes, alpha, scale, nt / 64, remap);
}

template <int B, bool F32>
tfp8_status launch_compress(const void *x, int64_t nb, float target, uint32_t flags,
                            uint8_t *codes, float *alpha, float *scale, hipStream_t st) {
  switch (flags) {
    case 0: return launch_compress_t<B, F32, 0>(x, nb, target, codes, alpha, scale, st);
    case kInt8: return launch_compress_t<B, F32, kInt8>(x, nb, target, codes, alpha, scale, st);
    case kNoRotation:
      return launch_compress_t<B, F32, kNoRotation>(x, nb, target, codes, alpha, scale, st);
    default:
      return launch_compress_t<B, F32, kInt8 | kNoRotation>(x, nb, target, codes, alpha, scale,
                                                            st);
  }
}

template <int B, bool F32, int FLAGS>
tfp8_status launch_decompress_t(const uint8_t *codes, const float *alpha, const float *scale,
                                int64_t nb, void *out, hipStream_t st) {
  constexpr bool ROT = !(FLAGS & kNoRotation);
  const float inv_sqrt_b = ROT ? (float)(1.0 / sqrt((double)B)) : 1.0f;
  constexpr int BPW = 64 / decompress_lanes(B);  // blocks per tile
  const int64_t tiles = (nb + BPW - 1) / BPW;
  const unsigned grid = grid_for(tiles, TFP8_DECOMPRESS_WGS_PER_CU);
  if ((int64_t)grid * (kThreads / 64) < tiles)  // capped launch: wavefronts loop over tiles
    return launch(k_decompress<B, F32, FLAGS, true>, grid, kThreads, st, codes, alpha, scale, nb,
                  inv_sqrt_b, out);
  return launch(k_decompress<B, F32, FLAGS, false>, grid, kThreads, st, codes, alpha, scale, nb,
                inv_sqrt_b, out);
}

template <int B, bool F32>
tfp8_status launch_decompress(const uint8_t *codes, const float *alpha, const float *scale,
                              int64_t nb, uint32_t flags, void *out, hipStream_t st) {
  switch (flags) {
    case 0: return launch_decompress_t<B, F32, 0>(codes, alpha, scale, nb, out, st);
    case kInt8: return launch_decompress_t<B, F32, kInt8>(codes, alpha, scale, nb, out, st);
    case kNoRotation:
      return launch_decompress_t<B, F32, kNoRotation>(codes, alpha, scale, nb, out, st);
    default:
      return launch_decompress_t<B, F32, kInt8 | kNoRotation>(codes, alpha, scale, nb, out, st);
  }
}

template <int B, int FLAGS>
tfp8_status launch_reduce_t(const uint8_t *codes, const float *alpha, const float *scale, int P,
                            int64_t cstride, int64_t astride, int64_t sstride, int64_t nb,
                            float target, uint8_t *codes_out, float *alpha_out, float *scale_out,
                            hipStream_t st) {
  // the reduce works on r = sum_p g_p dec(q_p) directly, with or without the rotation: its
  // energy is that of the sum, sum(r^2) = sum(z^2)
  const float TB = target * (float)B;
  constexpr int BPW = 64 / (B / 16);
  const unsigned grid = grid_for((nb + BPW - 1) / BPW, TFP8_REDUCE_WGS_PER_CU);
#define TFP8_LAUNCH_REDUCE(PB)                                                               \
  return launch(k_reduce<B, PB, FLAGS>, grid, kThreads, st, codes, alpha, scale, P, cstride,    \
                astride, sstride, nb, TB, codes_out, alpha_out, scale_out)
  switch (P) {
    case 1: TFP8_LAUNCH_REDUCE(1);
    case 2: TFP8_LAUNCH_REDUCE(2);
    case 4: TFP8_LAUNCH_REDUCE(4);
    case 8: TFP8_LAUNCH_REDUCE(8);
    default: TFP8_LAUNCH_REDUCE(0);
  }
#undef TFP8_LAUNCH_REDUCE
}

template <int B>
tfp8_status launch_reduce(const uint8_t *codes, const float *alpha, const float *scale, int P,
                          int64_t cstride, int64_t astride, int64_t sstride, int64_t nb,
                          float target, uint32_t flags, uint8_t *codes_out, float *alpha_out,
                          float *scale_out, hipStream_t st) {
  if (flags & kInt8)
    return launch_reduce_t<B, kInt8>(codes, alpha, scale, P, cstride, astride, sstride, nb, target,
                                     codes_out, alpha_out, scale_out, st);
  return launch_reduce_t<B, 0>(codes, alpha, scale, P, cstride, astride, sstride, nb, target,
                               codes_out, alpha_out, scale_out, st);
}

template <int B, bool F32, int FLAGS>
tfp8_status launch_accumulate_t(const uint8_t *codes, const float *alpha, const float *scale,
                                const void *grad, int64_t nb, float target, uint8_t *codes_out,
                                float *alpha_out, float *scale_out, hipStream_t st) {
  constexpr bool ROT = !(FLAGS & kNoRotation);
  const double Q = qmax_of<FLAGS>();
  const double TBBd = (double)target * B * (ROT ? B : 1);  // exact: powers of two
  const float TBB = (float)TBBd;
  const float sqrtTBB = (float)sqrt(TBBd);
  const double gscale = ROT ? sqrt((double)B) : 1.0;
  const double Cd = ROT ? Q * sqrt((double)B) : Q;
  const float C = (float)Cd, invC = (float)(1.0 / Cd);
  constexpr int BPW = 64 / lanes_per_block(B);  // blocks per tile
  const unsigned grid = grid_for((nb + BPW - 1) / BPW, TFP8_COMPRESS_WGS_PER_CU);
  const tfp8_status first =
      launch(k_accumulate<B, F32, FLAGS>, grid, kThreads, st, codes, alpha, scale, grad, nb, TBB,
             sqrtTBB, (float)gscale, C, invC, codes_out, alpha_out, scale_out);
  if (first != TFP8_OK) return first;
  // the set-aside blocks: codes and s from the inputs (untouched for them), -alpha from alpha_out
  const unsigned grid_fix =
      grid_for((nb + 64 * kFixRuns - 1) / (64 * kFixRuns), TFP8_ACCUMULATE_FIX_WGS_PER_CU);
  return launch(k_accumulate_fix<B, F32, FLAGS>, grid_fix, kThreads, st, codes, scale, grad, nb,
                TBB, C, gscale, codes_out, alpha_out, scale_out);
}

template <int B, bool F32>
tfp8_status launch_accumulate(const uint8_t *codes, const float *alpha, const float *scale,
                              const void *grad, int64_t nb, float target, uint32_t flags,
                              uint8_t *codes_out, float *alpha_out, float *scale_out,
                              hipStream_t st) {
#define TFP8_LAUNCH_ACCUMULATE(FL)                                                          \
  return launch_accumulate_t<B, F32, FL>(codes, alpha, scale, grad, nb, target, codes_out, \
                                         alpha_out, scale_out, st)
  switch (flags) {
    case 0: TFP8_LAUNCH_ACCUMULATE(0);
    case kInt8: TFP8_LAUNCH_ACCUMULATE(kInt8);
    case kNoRotation: TFP8_LAUNCH_ACCUMULATE(kNoRotation);
    default: TFP8_LAUNCH_ACCUMULATE(kInt8 | kNoRotation);
  }
#undef TFP8_LAUNCH_ACCUMULATE
}

}  // namespace

extern "C" {

int32_t tfp8_version(void) { return (1 << 16) | 3; }

const char *tfp8_status_string(tfp8_status status) {
  switch (status) {
    case TFP8_OK: return "ok";
    case TFP8_E_NULL: return "a required pointer is NULL";
    case TFP8_E_SIZE: return "n is negative, above 2^40, or not a multiple of the block size";
    case TFP8_E_BLOCK: return "unsupported block size (use 64, 128, 256 or 512)";
    case TFP8_E_DTYPE: return "unsupported dtype (use TFP8_BF16 or TFP8_F32)";
    case TFP8_E_ALIGN: return "misaligned pointer (16 bytes for data, 4 for scales)";
    case TFP8_E_ARG: return "bad argument (P, target, or overlapping buffers)";
    case TFP8_E_HIP: return "the HIP runtime rejected the kernel launch";
  }
  return "unknown status";
}

tfp8_status tfp8_compress_ex(const void *x, tfp8_dtype x_dtype, int64_t n, int32_t block,
                             float target, uint32_t flags, uint8_t *codes, float *alpha,
                             float *scale, void *stream) {
  if (!block_ok(block)) return TFP8_E_BLOCK;
  if (n < 0 || n > TFP8_MAX_N || n % block != 0) return TFP8_E_SIZE;
  if (x_dtype != TFP8_BF16 && x_dtype != TFP8_F32) return TFP8_E_DTYPE;
  if (!target_ok(target) || (flags & ~TFP8_FLAGS_ALL)) return TFP8_E_ARG;
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
#define TFP8_CASE(BB)                                                                         \
  case BB:                                                                                    \
    return f32 ? launch_compress<BB, true>(x, nb, target, flags, codes, alpha, scale, st)     \
               : launch_compress<BB, false>(x, nb, target, flags, codes, alpha, scale, st);
  switch (block) {
    TFP8_CASE(64)
    TFP8_CASE(128)
    TFP8_CASE(256)
    TFP8_CASE(512)
  }
#undef TFP8_CASE
  return TFP8_E_BLOCK;
}

tfp8_status tfp8_compress(const void *x, tfp8_dtype x_dtype, int64_t n, int32_t block, float target,
                          uint8_t *codes, float *alpha, float *scale, void *stream) {
  return tfp8_compress_ex(x, x_dtype, n, block, target, 0, codes, alpha, scale, stream);
}

tfp8_status tfp8_decompress_ex(const uint8_t *codes, const float *alpha, const float *scale,
                               int64_t n, int32_t block, uint32_t flags, void *out,
                               tfp8_dtype out_dtype, void *stream) {
  if (!block_ok(block)) return TFP8_E_BLOCK;
  if (n < 0 || n > TFP8_MAX_N || n % block != 0) return TFP8_E_SIZE;
  if (out_dtype != TFP8_BF16 && out_dtype != TFP8_F32) return TFP8_E_DTYPE;
  if (flags & ~TFP8_FLAGS_ALL) return TFP8_E_ARG;
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
#define TFP8_CASE(BB)                                                                        \
  case BB:                                                                                   \
    return f32 ? launch_decompress<BB, true>(codes, alpha, scale, nb, flags, out, st)        \
               : launch_decompress<BB, false>(codes, alpha, scale, nb, flags, out, st);
  switch (block) {
    TFP8_CASE(64)
    TFP8_CASE(128)
    TFP8_CASE(256)
    TFP8_CASE(512)
  }
#undef TFP8_CASE
  return TFP8_E_BLOCK;
}

tfp8_status tfp8_decompress(const uint8_t *codes, const float *alpha, const float *scale, int64_t n,
                            int32_t block, void *out, tfp8_dtype out_dtype, void *stream) {
  return tfp8_decompress_ex(codes, alpha, scale, n, block, 0, out, out_dtype, stream);
}

// The reduce entry points share this: contribution p at codes + p cstride (bytes) and
// alpha + p astride, scale + p sstride (floats); contiguous stacks have cstride = n and
// astride = sstride = n / block.  An input's span runs from its base to the end of its last
// contribution; no output may overlap any input span or another output.
static tfp8_status reduce_checked(const uint8_t *codes, int64_t cstride, const float *alpha,
                                  int64_t astride, const float *scale, int64_t sstride, int32_t P,
                                  int64_t n, int32_t block, float target, uint32_t flags,
                                  uint8_t *codes_out, float *alpha_out, float *scale_out,
                                  void *stream) {
  if (!block_ok(block)) return TFP8_E_BLOCK;
  if (n < 0 || n > TFP8_MAX_N || n % block != 0) return TFP8_E_SIZE;
  const int64_t nb = n / block;
  if (cstride > TFP8_MAX_N || astride > TFP8_MAX_N || sstride > TFP8_MAX_N) return TFP8_E_SIZE;
  if (P < 1 || P > 64 || !target_ok(target) || (flags & ~TFP8_FLAGS_ALL)) return TFP8_E_ARG;
  if (cstride < n || astride < nb || sstride < nb) return TFP8_E_ARG;  // rows would overlap
  if (n == 0) return TFP8_OK;
  if (!codes || !alpha || !scale || !codes_out || !alpha_out || !scale_out) return TFP8_E_NULL;
  if (!aligned(codes, 16) || !aligned(codes_out, 16) || !aligned(alpha, 4) || !aligned(scale, 4) ||
      !aligned(alpha_out, 4) || !aligned(scale_out, 4) || cstride % 16 != 0)
    return TFP8_E_ALIGN;
  const Range ins[3] = {range_of(codes, (int64_t)(P - 1) * cstride + n),
                        range_of(alpha, ((int64_t)(P - 1) * astride + nb) * 4),
                        range_of(scale, ((int64_t)(P - 1) * sstride + nb) * 4)};
  const Range outs[3] = {range_of(codes_out, n), range_of(alpha_out, nb * 4),
                         range_of(scale_out, nb * 4)};
  for (int i = 0; i < 3; ++i) {
    for (int k = 0; k < 3; ++k)
      if (overlap(outs[i], ins[k])) return TFP8_E_ARG;
    for (int k = i + 1; k < 3; ++k)
      if (overlap(outs[i], outs[k])) return TFP8_E_ARG;
  }
  hipStream_t st = (hipStream_t)stream;
#define TFP8_CASE(BB)                                                                          \
  case BB:                                                                                     \
    return launch_reduce<BB>(codes, alpha, scale, P, cstride, astride, sstride, nb, target,    \
                             flags, codes_out, alpha_out, scale_out, st);
  switch (block) {
    TFP8_CASE(64)
    TFP8_CASE(128)
    TFP8_CASE(256)
    TFP8_CASE(512)
  }
#undef TFP8_CASE
  return TFP8_E_BLOCK;
}

tfp8_status tfp8_reduce_ex(const uint8_t *codes, const float *alpha, const float *scale, int32_t P,
                           int64_t n, int32_t block, float target, uint32_t flags,
                           uint8_t *codes_out, float *alpha_out, float *scale_out, void *stream) {
  const int64_t nb = block_ok(block) ? n / block : 0;
  return reduce_checked(codes, n, alpha, nb, scale, nb, P, n, block, target, flags, codes_out,
                        alpha_out, scale_out, stream);
}

tfp8_status tfp8_reduce_strided(const uint8_t *codes, int64_t codes_stride, const float *alpha,
                                int64_t alpha_stride, const float *scale, int64_t scale_stride,
                                int32_t P, int64_t n, int32_t block, float target, uint32_t flags,
                                uint8_t *codes_out, float *alpha_out, float *scale_out,
                                void *stream) {
  return reduce_checked(codes, codes_stride, alpha, alpha_stride, scale, scale_stride, P, n, block,
                        target, flags, codes_out, alpha_out, scale_out, stream);
}

tfp8_status tfp8_reduce_fp8(const uint8_t *codes, const float *alpha, const float *scale, int32_t P,
                            int64_t n, int32_t block, float target, uint8_t *codes_out,
                            float *alpha_out, float *scale_out, void *stream) {
  return tfp8_reduce_ex(codes, alpha, scale, P, n, block, target, 0, codes_out, alpha_out,
                        scale_out, stream);
}

tfp8_status tfp8_accumulate(const uint8_t *codes, const float *alpha, const float *scale,
                            const void *grad, tfp8_dtype grad_dtype, int64_t n, int32_t block,
                            float target, uint32_t flags, uint8_t *codes_out, float *alpha_out,
                            float *scale_out, void *stream) {
  if (!block_ok(block)) return TFP8_E_BLOCK;
  if (n < 0 || n > TFP8_MAX_N || n % block != 0) return TFP8_E_SIZE;
  if (grad_dtype != TFP8_BF16 && grad_dtype != TFP8_F32) return TFP8_E_DTYPE;
  if (!target_ok(target) || (flags & ~TFP8_FLAGS_ALL)) return TFP8_E_ARG;
  if (n == 0) return TFP8_OK;
  if (!codes || !alpha || !scale || !grad || !codes_out || !alpha_out || !scale_out)
    return TFP8_E_NULL;
  if (!aligned(codes, 16) || !aligned(codes_out, 16) || !aligned(grad, 16) || !aligned(alpha, 4) ||
      !aligned(scale, 4) || !aligned(alpha_out, 4) || !aligned(scale_out, 4))
    return TFP8_E_ALIGN;
  const int64_t nb = n / block;
  // In place is allowed: each output may be exactly its input.  Any other overlap is rejected.
  const Range rq = range_of(codes, n), ra = range_of(alpha, nb * 4), rs = range_of(scale, nb * 4),
              rg = range_of(grad, n * (grad_dtype == TFP8_F32 ? 4 : 2));
  const Range oq = range_of(codes_out, n), oa = range_of(alpha_out, nb * 4),
              os = range_of(scale_out, nb * 4);
  const Range outs[3] = {oq, oa, os};
  const Range same[3] = {rq, ra, rs};
  const Range ins[4] = {rq, ra, rs, rg};
  for (int i = 0; i < 3; ++i) {
    for (int k = 0; k < 4; ++k)
      if (overlap(outs[i], ins[k]) && !(k == i && outs[i].lo == same[i].lo)) return TFP8_E_ARG;
    for (int k = i + 1; k < 3; ++k)
      if (overlap(outs[i], outs[k])) return TFP8_E_ARG;
  }
  hipStream_t st = (hipStream_t)stream;
  const bool f32 = grad_dtype == TFP8_F32;
#define TFP8_CASE(BB)                                                                          \
  case BB:                                                                                     \
    return f32 ? launch_accumulate<BB, true>(codes, alpha, scale, grad, nb, target, flags,     \
                                             codes_out, alpha_out, scale_out, st)              \
               : launch_accumulate<BB, false>(codes, alpha, scale, grad, nb, target, flags,    \
                                              codes_out, alpha_out, scale_out, st);
  switch (block) {
    TFP8_CASE(64)
    TFP8_CASE(128)
    TFP8_CASE(256)
    TFP8_CASE(512)
  }
#undef TFP8_CASE
  return TFP8_E_BLOCK;
}

}  // extern "C"
