/*
 * tfp8_oracle.h - plain FP64 CPU oracle for TACO-style FP8 (ASH + DS) block compression.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or calls this
 * code; only the test suite, the smoke check and the benchmark's CPU-baseline leg do.  It is
 * slow on purpose: one block at a time, every step written out, float64 everywhere, rounding
 * only where a value is stored (fp32 scales, E4M3 codes, the output dtype).
 *
 * What it computes follows the TACO summary page ("TACO: Efficient Communication Compression
 * of Intermediate Tensors for Scalable Tensor-Parallel LLM Training"): FP8 E4M3 as the code
 * format (section 2.A), the adaptive scale-Hadamard transform (section 2.B.1), dual-scale
 * quantization and its inverse (section 2.B.2); and the local reduce of the AGoQ summary page
 * ("AGoQ: Activation and Gradient Quantization for Memory-Efficient Distributed Training of
 * LLMs", section 2.B): dequantize every contribution, sum, requantize.
 *
 * All pointers are host pointers.  Buffers are caller-owned.  Every function returns 0 on
 * success or a negative TFP8_REF_E_* code on bad arguments and then writes nothing.
 */
#ifndef TFP8_ORACLE_H
#define TFP8_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TFP8_REF_OK = 0,
  TFP8_REF_E_NULL = -1,  /* a required pointer is NULL */
  TFP8_REF_E_SIZE = -2,  /* n < 0 or n % block != 0 */
  TFP8_REF_E_BLOCK = -3, /* block is not a power of two in [2, 4096] */
  TFP8_REF_E_DTYPE = -4, /* dtype is neither 0 (bf16) nor 1 (fp32) */
  TFP8_REF_E_ARG = -6    /* P < 1, or target not finite in [2^-64, 2^64] */
};

enum { TFP8_REF_BF16 = 0, TFP8_REF_F32 = 1 };

/* Variant flags of the *_ex functions (0 = the method as defined on the TACO page):
 *   TFP8_REF_INT8         codes are int8 (two's complement, round to nearest even, saturating
 *                         at +-127) with Q_max = 127: the INT8 fallback the TACO page mentions for
 *                         hardware without FP8 (section 5);
 *   TFP8_REF_NO_ROTATION  the Hadamard rotation is left out (identity), for ablations. */
enum { TFP8_REF_INT8 = 1, TFP8_REF_NO_ROTATION = 2 };

/* E4M3FN (max 448, no infinities, 0x7F/0xFF NaN): encode v with round-to-nearest-even,
 * saturating at +-448, sign taken from v (so a tiny negative gives 0x80). */
uint8_t tfp8_ref_e4m3_encode(double v);
/* Exact value of an E4M3FN code; NaN for 0x7F and 0xFF. */
double tfp8_ref_e4m3_decode(uint8_t code);
/* Round a float64 straight to bfloat16 (nearest-even, one rounding) and return its bits. */
uint16_t tfp8_ref_round_bf16(double v);

/* Sylvester Hadamard entry H[i][j] = (-1)^popcount(i & j). */
int tfp8_ref_hadamard_entry(int64_t i, int64_t j);
/* Unnormalised fast Walsh-Hadamard transform in place: v <- H v (natural order). */
void tfp8_ref_fwht(double *v, int64_t len);
/* The same product by the explicit matrix, O(len^2): out <- H v. */
void tfp8_ref_hadamard_dense(const double *v, int64_t len, double *out);

/* Compress n elements (bf16 bits or fp32) in blocks of `block`.
 * Outputs: codes[n], alpha[n/block], scale[n/block].  If `quot` is not NULL it receives the
 * exact (float64) quotient y_i / s_k that each code rounds. */
int tfp8_ref_compress(const void *x, int x_dtype, int64_t n, int block, float target,
                      uint8_t *codes, float *alpha, float *scale, double *quot);

/* Decompress to bf16 bits or fp32 (out_dtype), one rounding from the float64 result. */
int tfp8_ref_decompress(const uint8_t *codes, const float *alpha, const float *scale, int64_t n,
                        int block, void *out, int out_dtype);

/* Float64 reconstruction with no rounding of the result (for error identities). */
int tfp8_ref_decompress_f64(const uint8_t *codes, const float *alpha, const float *scale, int64_t n,
                            int block, double *out);

/* Compress with the E4M3 rounding bypassed: t[n] = y/s exactly (float64); alpha and scale are
 * rounded to fp32 as usual.  Used to show the transform is exactly invertible. */
int tfp8_ref_compress_unrounded(const void *x, int x_dtype, int64_t n, int block, float target,
                                double *t, float *alpha, float *scale);
/* Inverse of the above: out = H (s * t) / (sqrt(block) * alpha), float64. */
int tfp8_ref_decompress_unrounded(const double *t, const float *alpha, const float *scale,
                                  int64_t n, int block, double *out);

/* Local reduce of P contributions stacked [P][n] (codes) and [P][n/block] (scales), by the
 * definition: reconstruct every contribution in float64, sum, compress the sum. */
int tfp8_ref_reduce_fp8(const uint8_t *codes, const float *alpha, const float *scale, int P,
                        int64_t n, int block, float target, uint8_t *codes_out, float *alpha_out,
                        float *scale_out, double *quot);

/* The same reduce computed in the rotated domain (no Hadamard): r = sum_p (s_p/alpha_p) dec(q_p),
 * requantised directly.  A second, independent route used to cross-check the first. */
int tfp8_ref_reduce_fp8_rotated(const uint8_t *codes, const float *alpha, const float *scale,
                                int P, int64_t n, int block, float target, uint8_t *codes_out,
                                float *alpha_out, float *scale_out, double *quot);

/* Variants selected by `flags` (TFP8_REF_INT8, TFP8_REF_NO_ROTATION); same arguments otherwise. */
uint8_t tfp8_ref_int8_encode(double v);
double tfp8_ref_int8_decode(uint8_t code);
int tfp8_ref_compress_ex(const void *x, int x_dtype, int64_t n, int block, float target, int flags,
                         uint8_t *codes, float *alpha, float *scale, double *quot);
int tfp8_ref_decompress_ex(const uint8_t *codes, const float *alpha, const float *scale, int64_t n,
                           int block, int flags, void *out, int out_dtype);
int tfp8_ref_decompress_f64_ex(const uint8_t *codes, const float *alpha, const float *scale,
                               int64_t n, int block, int flags, double *out);
int tfp8_ref_reduce_ex(const uint8_t *codes, const float *alpha, const float *scale, int P,
                       int64_t n, int block, float target, int flags, uint8_t *codes_out,
                       float *alpha_out, float *scale_out, double *quot);
int tfp8_ref_reduce_rotated_ex(const uint8_t *codes, const float *alpha, const float *scale, int P,
                               int64_t n, int block, float target, int flags, uint8_t *codes_out,
                               float *alpha_out, float *scale_out, double *quot);

/* Local gradient accumulation ("AGoQ: Activation and Gradient Quantization for Memory-Efficient
 * Distributed Training of LLMs", section 2.B): the compressed main gradient (codes, alpha, scale)
 * is reconstructed, the dense local gradient grad[n] (bf16 bits or fp32) is added, and the sum is
 * compressed again with the same block, target and flags.  By the definition (float64). */
int tfp8_ref_accumulate_ex(const uint8_t *codes, const float *alpha, const float *scale,
                           const void *grad, int grad_dtype, int64_t n, int block, float target,
                           int flags, uint8_t *codes_out, float *alpha_out, float *scale_out,
                           double *quot);
/* The same sum formed in the rotated domain: H z = sqrt(B) (s/alpha) dec(q) + H g (unnormalised
 * H), so only the dense gradient is transformed.  A second route used to cross-check the first. */
int tfp8_ref_accumulate_rotated_ex(const uint8_t *codes, const float *alpha, const float *scale,
                                   const void *grad, int grad_dtype, int64_t n, int block,
                                   float target, int flags, uint8_t *codes_out, float *alpha_out,
                                   float *scale_out, double *quot);

/* Threads used by the block loops (OpenMP); returns the count in effect. */
int tfp8_ref_set_threads(int threads);

#ifdef __cplusplus
}
#endif
#endif
