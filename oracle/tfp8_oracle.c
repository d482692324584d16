/*
 * tfp8_oracle.c - plain FP64 CPU oracle for TACO-style FP8 (ASH + DS) block compression.
 *
 * TEST INFRASTRUCTURE ONLY (see tfp8_oracle.h): used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product library.  It shares no code, header,
 * table or constant with the HIP path.
 *
 * Sources of each step (page titles as printed; sections as numbered on each page):
 *   [TACO] "TACO: Efficient Communication Compression of Intermediate Tensors for Scalable
 *          Tensor-Parallel LLM Training".
 *   [AGoQ] "AGoQ: Activation and Gradient Quantization for Memory-Efficient Distributed
 *          Training of LLMs".
 *
 * Readings where the pages leave a step open:
 *   - a block is `block` consecutive elements of the flat buffer; the Hadamard size is `block`;
 *   - the block's second moment, its energy, is the raw mean of squares m2 = sum(v^2)/block;
 *   - the prescale brings that energy to the target: alpha = sqrt(target/m2), clamped to
 *     [2^-126, 2^126] so that alpha and 1/alpha are normal fp32 numbers;
 *   - the rotation is the Sylvester Hadamard in natural order, normalised by 1/sqrt(block),
 *     with no random signs;
 *   - the post-scale is s = max|y| / 448 (448 = largest E4M3FN value; 127 for the INT8 codes);
 *   - codes are OCP E4M3FN, round-to-nearest-even, saturating, sign kept on zero;
 *   - an all-zero block (tested on max|v|, not on m2) stores alpha = 1, s = 0, codes 0x00 and
 *     reconstructs to +0;
 *   - both scales are stored as fp32 and every later step uses the stored values;
 *   - the INT8 variant uses two's-complement codes, round-to-nearest-even, saturating at +-127,
 *     with Q_max = 127; the no-rotation variant replaces H by the identity;
 *   - the local accumulation reconstructs the main gradient, adds the local gradient and
 *     compresses the sum with the same block, target and variant.
 *
 * Parity unpinned: the default target (1), the alpha clamp bounds and the Sylvester order
 * without random signs are conventions the pages do not fix, so no test can tie them to the
 * pages; the tests pin everything the oracle computes given them.
 */
#include "tfp8_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

int tfp8_ref_set_threads(int threads) {
  if (threads < 1) threads = 1;
  g_threads = threads;
  return g_threads;
}

/* ---------------------------------------------------------------------------------------- */
/* E4M3FN code ([TACO] section 2.A names E4M3; the format's layout is OCP's 8-bit float:      */
/* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, 0x7F/0xFF NaN).  */

double tfp8_ref_e4m3_decode(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);              /* subnormal: m * 2^-9 */
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);       /* normal: (1 + m/8) * 2^(e-7) */
  return sign ? -mag : mag;
}

uint8_t tfp8_ref_e4m3_encode(double v) {
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs(v);
  if (!(a <= 448.0)) return sign | 0x7E;     /* saturate (never reached by compress) */
  if (a < 0x1p-6) {
    /* below the smallest normal the grid is uniform with step 2^-9; k = 8 is the code of
       2^-6 itself (exponent field 1, mantissa 0), so the code equals k. */
    double k = nearbyint(a * 512.0);         /* exact scaling, then round-half-even */
    return sign | (uint8_t)k;
  }
  int ex;
  frexp(a, &ex);                             /* a = f * 2^ex, f in [0.5, 1) */
  int E = ex - 1;                            /* floor(log2 a), in [-6, 8] */
  double k = nearbyint(ldexp(a, 3 - E));     /* significand in eighths, in [8, 16] */
  if (k == 16.0) {
    E += 1;
    k = 8.0;
  }
  return sign | (uint8_t)(((E + 7) << 3) | ((int)k - 8));
}

uint16_t tfp8_ref_round_bf16(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex);
  int E = ex - 1;
  /* bfloat16 keeps 8 significant bits; below 2^-126 the grid is uniform with step 2^-133 */
  double step = (E < -126) ? 0x1p-133 : ldexp(1.0, E - 7);
  double r = nearbyint(a / step) * step;     /* one rounding, half to even */
  float f = (float)r;                        /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return sign | (uint16_t)(u >> 16);
}

/* INT8 code for the fallback the TACO page keeps for hardware without FP8 (section 5): a
   two's complement byte, round to nearest even, saturating at +-127 (symmetric, so -128 is
   never produced; it still decodes to -128). */
uint8_t tfp8_ref_int8_encode(double v) {
  double k = nearbyint(v);
  if (k > 127.0) k = 127.0;
  if (k < -127.0) k = -127.0;
  return (uint8_t)(int8_t)k;
}

double tfp8_ref_int8_decode(uint8_t code) { return (double)(int8_t)code; }

static double code_value(uint8_t code, int flags) {
  return (flags & TFP8_REF_INT8) ? tfp8_ref_int8_decode(code) : tfp8_ref_e4m3_decode(code);
}

static uint8_t code_encode(double t, int flags) {
  return (flags & TFP8_REF_INT8) ? tfp8_ref_int8_encode(t) : tfp8_ref_e4m3_encode(t);
}

/* Q_max: the largest code value the post-scale maps the block's peak to. */
static double code_qmax(int flags) { return (flags & TFP8_REF_INT8) ? 127.0 : 448.0; }

/* ---------------------------------------------------------------------------------------- */
/* Hadamard ([TACO] section 2.B.1: an orthogonal Hadamard rotation).                          */

int tfp8_ref_hadamard_entry(int64_t i, int64_t j) {
  return (__builtin_popcountll((unsigned long long)(i & j)) & 1) ? -1 : 1;
}

void tfp8_ref_fwht(double *v, int64_t len) {
  for (int64_t h = 1; h < len; h <<= 1)
    for (int64_t i = 0; i < len; i += 2 * h)
      for (int64_t j = i; j < i + h; ++j) {
        double a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
}

void tfp8_ref_hadamard_dense(const double *v, int64_t len, double *out) {
  for (int64_t i = 0; i < len; ++i) {
    double acc = 0.0;
    for (int64_t j = 0; j < len; ++j) acc += tfp8_ref_hadamard_entry(i, j) * v[j];
    out[i] = acc;
  }
}

/* ---------------------------------------------------------------------------------------- */
/* argument checks                                                                            */

static int check_block(int block) {
  if (block < 2 || block > 4096 || (block & (block - 1)) != 0) return TFP8_REF_E_BLOCK;
  return TFP8_REF_OK;
}

static int check_common(int64_t n, int block) {
  int st = check_block(block);
  if (st) return st;
  if (n < 0 || n % block != 0) return TFP8_REF_E_SIZE;
  return TFP8_REF_OK;
}

static int check_target(float target) {
  if (!isfinite(target) || !(target >= 0x1p-64f) || !(target <= 0x1p64f)) return TFP8_REF_E_ARG;
  return TFP8_REF_OK;
}

static double load_elem(const void *x, int dtype, int64_t i) {
  if (dtype == TFP8_REF_F32) return (double)((const float *)x)[i];
  uint32_t u = (uint32_t)((const uint16_t *)x)[i] << 16;   /* bf16 widens exactly */
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ---------------------------------------------------------------------------------------- */
/* ASH + DS on one block of float64 values v[0..B) ([TACO] sections 2.B.1 and 2.B.2).        */
/* If `quot` is not NULL it receives y_i / s; if `codes` is NULL the rounding is skipped.     */

static void compress_block(const double *v, int B, double T, int flags, uint8_t *codes,
                           float *alpha_out, float *scale_out, double *quot) {
  double ax = 0.0;
  for (int i = 0; i < B; ++i) ax = fmax(ax, fabs(v[i]));
  if (ax == 0.0) { /* all-zero block: nothing to scale */
    *alpha_out = 1.0f;
    *scale_out = 0.0f;
    for (int i = 0; i < B; ++i) {
      if (codes) codes[i] = 0x00;
      if (quot) quot[i] = 0.0;
    }
    return;
  }
  /* second moment (energy) of the block */
  double sumsq = 0.0;
  for (int i = 0; i < B; ++i) sumsq += v[i] * v[i];
  double m2 = sumsq / B;
  /* adaptive prescale that brings the energy to the target level */
  double a = sqrt(T / m2);
  a = fmin(fmax(a, 0x1p-126), 0x1p126);
  float alpha = (float)a;
  /* orthogonal Hadamard rotation of the prescaled block (left out for the ablation variant) */
  double *y = (double *)malloc(sizeof(double) * (size_t)B);
  for (int i = 0; i < B; ++i) y[i] = (double)alpha * v[i];
  if (!(flags & TFP8_REF_NO_ROTATION)) {
    tfp8_ref_fwht(y, B);
    double rootB = sqrt((double)B);
    for (int i = 0; i < B; ++i) y[i] = y[i] / rootB;
  }
  /* post-scale: largest rotated magnitude lands on Q_max (448 for E4M3) */
  double my = 0.0;
  for (int i = 0; i < B; ++i) my = fmax(my, fabs(y[i]));
  float s = (float)(my / code_qmax(flags));
  for (int i = 0; i < B; ++i) {
    double t = y[i] / (double)s;
    if (quot) quot[i] = t;
    if (codes) codes[i] = code_encode(t, flags);
  }
  *alpha_out = alpha;
  *scale_out = s;
  free(y);
}

/* Inverse of one block from the code values c_j = dec(q_j) (or unrounded quotients):
   x_i = (1/sqrt(B)) * sum_j H[i][j] (s * c_j) / alpha ([TACO] section 2.B.2, reconstruction
   with both scales; H is symmetric and (H/sqrt(B))^2 = I). */
static void decompress_block(const double *cval, float alpha, float scale, int B, int flags,
                             double *out) {
  if (scale == 0.0f) {
    for (int i = 0; i < B; ++i) out[i] = 0.0;
    return;
  }
  for (int i = 0; i < B; ++i) out[i] = (double)scale * cval[i];
  if (!(flags & TFP8_REF_NO_ROTATION)) {
    tfp8_ref_fwht(out, B);
    double rootB = sqrt((double)B);
    for (int i = 0; i < B; ++i) out[i] = out[i] / rootB;
  }
  for (int i = 0; i < B; ++i) out[i] = out[i] / (double)alpha;
}

/* ---------------------------------------------------------------------------------------- */

static int check_flags(int flags) {
  return (flags & ~(TFP8_REF_INT8 | TFP8_REF_NO_ROTATION)) ? TFP8_REF_E_ARG : TFP8_REF_OK;
}

int tfp8_ref_compress_ex(const void *x, int x_dtype, int64_t n, int block, float target, int flags,
                         uint8_t *codes, float *alpha, float *scale, double *quot) {
  int st = check_common(n, block);
  if (st) return st;
  if (x_dtype != TFP8_REF_BF16 && x_dtype != TFP8_REF_F32) return TFP8_REF_E_DTYPE;
  if ((st = check_target(target)) || (st = check_flags(flags))) return st;
  if (n == 0) return TFP8_REF_OK;
  if (!x || !codes || !alpha || !scale) return TFP8_REF_E_NULL;
  int64_t nb = n / block;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t k = 0; k < nb; ++k) {
    double *v = (double *)malloc(sizeof(double) * (size_t)block);
    for (int i = 0; i < block; ++i) v[i] = load_elem(x, x_dtype, k * block + i);
    compress_block(v, block, (double)target, flags, codes + k * block, alpha + k, scale + k,
                   quot ? quot + k * block : NULL);
    free(v);
  }
  return TFP8_REF_OK;
}

int tfp8_ref_compress(const void *x, int x_dtype, int64_t n, int block, float target,
                      uint8_t *codes, float *alpha, float *scale, double *quot) {
  return tfp8_ref_compress_ex(x, x_dtype, n, block, target, 0, codes, alpha, scale, quot);
}

int tfp8_ref_compress_unrounded(const void *x, int x_dtype, int64_t n, int block, float target,
                                double *t, float *alpha, float *scale) {
  int st = check_common(n, block);
  if (st) return st;
  if (x_dtype != TFP8_REF_BF16 && x_dtype != TFP8_REF_F32) return TFP8_REF_E_DTYPE;
  if ((st = check_target(target))) return st;
  if (n == 0) return TFP8_REF_OK;
  if (!x || !t || !alpha || !scale) return TFP8_REF_E_NULL;
  int64_t nb = n / block;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t k = 0; k < nb; ++k) {
    double *v = (double *)malloc(sizeof(double) * (size_t)block);
    for (int i = 0; i < block; ++i) v[i] = load_elem(x, x_dtype, k * block + i);
    compress_block(v, block, (double)target, 0, NULL, alpha + k, scale + k, t + k * block);
    free(v);
  }
  return TFP8_REF_OK;
}

int tfp8_ref_decompress_f64_ex(const uint8_t *codes, const float *alpha, const float *scale,
                               int64_t n, int block, int flags, double *out) {
  int st = check_common(n, block);
  if (st || (st = check_flags(flags))) return st;
  if (n == 0) return TFP8_REF_OK;
  if (!codes || !alpha || !scale || !out) return TFP8_REF_E_NULL;
  int64_t nb = n / block;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t k = 0; k < nb; ++k) {
    double *c = (double *)malloc(sizeof(double) * (size_t)block);
    for (int i = 0; i < block; ++i) c[i] = code_value(codes[k * block + i], flags);
    decompress_block(c, alpha[k], scale[k], block, flags, out + k * block);
    free(c);
  }
  return TFP8_REF_OK;
}

int tfp8_ref_decompress_f64(const uint8_t *codes, const float *alpha, const float *scale, int64_t n,
                            int block, double *out) {
  return tfp8_ref_decompress_f64_ex(codes, alpha, scale, n, block, 0, out);
}

int tfp8_ref_decompress_ex(const uint8_t *codes, const float *alpha, const float *scale, int64_t n,
                           int block, int flags, void *out, int out_dtype) {
  int st = check_common(n, block);
  if (st || (st = check_flags(flags))) return st;
  if (out_dtype != TFP8_REF_BF16 && out_dtype != TFP8_REF_F32) return TFP8_REF_E_DTYPE;
  if (n == 0) return TFP8_REF_OK;
  if (!codes || !alpha || !scale || !out) return TFP8_REF_E_NULL;
  int64_t nb = n / block;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t k = 0; k < nb; ++k) {
    double *c = (double *)malloc(sizeof(double) * (size_t)block);
    double *r = (double *)malloc(sizeof(double) * (size_t)block);
    for (int i = 0; i < block; ++i) c[i] = code_value(codes[k * block + i], flags);
    decompress_block(c, alpha[k], scale[k], block, flags, r);
    for (int i = 0; i < block; ++i) {
      if (out_dtype == TFP8_REF_F32)
        ((float *)out)[k * block + i] = (float)r[i];
      else
        ((uint16_t *)out)[k * block + i] = tfp8_ref_round_bf16(r[i]);
    }
    free(c);
    free(r);
  }
  return TFP8_REF_OK;
}

int tfp8_ref_decompress(const uint8_t *codes, const float *alpha, const float *scale, int64_t n,
                        int block, void *out, int out_dtype) {
  return tfp8_ref_decompress_ex(codes, alpha, scale, n, block, 0, out, out_dtype);
}

int tfp8_ref_decompress_unrounded(const double *t, const float *alpha, const float *scale,
                                  int64_t n, int block, double *out) {
  int st = check_common(n, block);
  if (st) return st;
  if (n == 0) return TFP8_REF_OK;
  if (!t || !alpha || !scale || !out) return TFP8_REF_E_NULL;
  int64_t nb = n / block;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t k = 0; k < nb; ++k) decompress_block(t + k * block, alpha[k], scale[k], block, 0, out + k * block);
  return TFP8_REF_OK;
}

/* ---------------------------------------------------------------------------------------- */
/* Local reduce ([AGoQ] section 2.B: dequantize the received contributions to FP32, sum,     */
/* quantize again; [TACO] section 2.B.3 places this step between ReduceScatter and           */
/* AllGather).  The oracle sums in float64.                                                  */

static int check_reduce(const uint8_t *codes, const float *alpha, const float *scale, int P,
                        int64_t n, int block, float target, int flags, uint8_t *codes_out,
                        float *alpha_out, float *scale_out) {
  int st = check_common(n, block);
  if (st) return st;
  if (P < 1) return TFP8_REF_E_ARG;
  if ((st = check_target(target)) || (st = check_flags(flags))) return st;
  if (n == 0) return TFP8_REF_OK;
  if (!codes || !alpha || !scale || !codes_out || !alpha_out || !scale_out) return TFP8_REF_E_NULL;
  return TFP8_REF_OK;
}

int tfp8_ref_reduce_ex(const uint8_t *codes, const float *alpha, const float *scale, int P,
                       int64_t n, int block, float target, int flags, uint8_t *codes_out,
                       float *alpha_out, float *scale_out, double *quot) {
  int st = check_reduce(codes, alpha, scale, P, n, block, target, flags, codes_out, alpha_out,
                        scale_out);
  if (st || n == 0) return st;
  int64_t nb = n / block;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t k = 0; k < nb; ++k) {
    double *z = (double *)calloc((size_t)block, sizeof(double));
    double *c = (double *)malloc(sizeof(double) * (size_t)block);
    double *xh = (double *)malloc(sizeof(double) * (size_t)block);
    for (int p = 0; p < P; ++p) {
      const uint8_t *q = codes + (int64_t)p * n + k * block;
      for (int i = 0; i < block; ++i) c[i] = code_value(q[i], flags);
      decompress_block(c, alpha[(int64_t)p * nb + k], scale[(int64_t)p * nb + k], block, flags, xh);
      for (int i = 0; i < block; ++i) z[i] += xh[i];
    }
    compress_block(z, block, (double)target, flags, codes_out + k * block, alpha_out + k,
                   scale_out + k, quot ? quot + k * block : NULL);
    free(z);
    free(c);
    free(xh);
  }
  return TFP8_REF_OK;
}

int tfp8_ref_reduce_fp8(const uint8_t *codes, const float *alpha, const float *scale, int P,
                        int64_t n, int block, float target, uint8_t *codes_out, float *alpha_out,
                        float *scale_out, double *quot) {
  return tfp8_ref_reduce_ex(codes, alpha, scale, P, n, block, target, 0, codes_out, alpha_out,
                            scale_out, quot);
}

int tfp8_ref_reduce_rotated_ex(const uint8_t *codes, const float *alpha, const float *scale, int P,
                               int64_t n, int block, float target, int flags, uint8_t *codes_out,
                               float *alpha_out, float *scale_out, double *quot) {
  int st = check_reduce(codes, alpha, scale, P, n, block, target, flags, codes_out, alpha_out,
                        scale_out);
  if (st || n == 0) return st;
  int64_t nb = n / block;
  double T = (double)target;
  double Q = code_qmax(flags);
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t k = 0; k < nb; ++k) {
    /* The sum z = sum_p H(s_p dec q_p)/(sqrt(B) alpha_p) equals H r / sqrt(B) with
       r = sum_p (s_p/alpha_p) dec(q_p).  Because H/sqrt(B) is orthogonal and its own inverse:
       mean(z^2) = mean(r^2), z = 0 exactly when r = 0, and the rotated prescaled sum is
       y = (1/sqrt(B)) H (alpha z) = alpha r.  So no Hadamard is applied at all.  (Without the
       rotation, z = r directly and the same holds.) */
    double *r = (double *)calloc((size_t)block, sizeof(double));
    for (int p = 0; p < P; ++p) {
      float s = scale[(int64_t)p * nb + k];
      if (s == 0.0f) continue;
      double g = (double)s / (double)alpha[(int64_t)p * nb + k];
      const uint8_t *q = codes + (int64_t)p * n + k * block;
      for (int i = 0; i < block; ++i) r[i] += g * code_value(q[i], flags);
    }
    double ar = 0.0, sumsq = 0.0;
    for (int i = 0; i < block; ++i) {
      ar = fmax(ar, fabs(r[i]));
      sumsq += r[i] * r[i];
    }
    uint8_t *qo = codes_out + k * block;
    if (ar == 0.0) {
      alpha_out[k] = 1.0f;
      scale_out[k] = 0.0f;
      for (int i = 0; i < block; ++i) {
        qo[i] = 0x00;
        if (quot) quot[k * block + i] = 0.0;
      }
      free(r);
      continue;
    }
    double a = sqrt(T / (sumsq / block));
    a = fmin(fmax(a, 0x1p-126), 0x1p126);
    float alpha2 = (float)a;
    float s2 = (float)((double)alpha2 * ar / Q);
    for (int i = 0; i < block; ++i) {
      double t = (double)alpha2 * r[i] / (double)s2;
      if (quot) quot[k * block + i] = t;
      qo[i] = code_encode(t, flags);
    }
    alpha_out[k] = alpha2;
    scale_out[k] = s2;
    free(r);
  }
  return TFP8_REF_OK;
}

int tfp8_ref_reduce_fp8_rotated(const uint8_t *codes, const float *alpha, const float *scale,
                                int P, int64_t n, int block, float target, uint8_t *codes_out,
                                float *alpha_out, float *scale_out, double *quot) {
  return tfp8_ref_reduce_rotated_ex(codes, alpha, scale, P, n, block, target, 0, codes_out,
                                    alpha_out, scale_out, quot);
}

/* ---------------------------------------------------------------------------------------- */
/* Local gradient accumulation ([AGoQ] section 2.B: dequantize the FP8 main gradient, add the  */
/* new local gradient, quantize the sum again).  The oracle forms the sum in float64.          */

static int check_accumulate(const uint8_t *codes, const float *alpha, const float *scale,
                            const void *grad, int grad_dtype, int64_t n, int block, float target,
                            int flags, uint8_t *codes_out, float *alpha_out, float *scale_out) {
  int st = check_common(n, block);
  if (st) return st;
  if (grad_dtype != TFP8_REF_BF16 && grad_dtype != TFP8_REF_F32) return TFP8_REF_E_DTYPE;
  if ((st = check_target(target)) || (st = check_flags(flags))) return st;
  if (n == 0) return TFP8_REF_OK;
  if (!codes || !alpha || !scale || !grad || !codes_out || !alpha_out || !scale_out)
    return TFP8_REF_E_NULL;
  return TFP8_REF_OK;
}

int tfp8_ref_accumulate_ex(const uint8_t *codes, const float *alpha, const float *scale,
                           const void *grad, int grad_dtype, int64_t n, int block, float target,
                           int flags, uint8_t *codes_out, float *alpha_out, float *scale_out,
                           double *quot) {
  int st = check_accumulate(codes, alpha, scale, grad, grad_dtype, n, block, target, flags,
                            codes_out, alpha_out, scale_out);
  if (st || n == 0) return st;
  int64_t nb = n / block;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t k = 0; k < nb; ++k) {
    double *c = (double *)malloc(sizeof(double) * (size_t)block);
    double *z = (double *)malloc(sizeof(double) * (size_t)block);
    for (int i = 0; i < block; ++i) c[i] = code_value(codes[k * block + i], flags);
    decompress_block(c, alpha[k], scale[k], block, flags, z);
    for (int i = 0; i < block; ++i) z[i] += load_elem(grad, grad_dtype, k * block + i);
    compress_block(z, block, (double)target, flags, codes_out + k * block, alpha_out + k,
                   scale_out + k, quot ? quot + k * block : NULL);
    free(c);
    free(z);
  }
  return TFP8_REF_OK;
}

int tfp8_ref_accumulate_rotated_ex(const uint8_t *codes, const float *alpha, const float *scale,
                                   const void *grad, int grad_dtype, int64_t n, int block,
                                   float target, int flags, uint8_t *codes_out, float *alpha_out,
                                   float *scale_out, double *quot) {
  int st = check_accumulate(codes, alpha, scale, grad, grad_dtype, n, block, target, flags,
                            codes_out, alpha_out, scale_out);
  if (st || n == 0) return st;
  int64_t nb = n / block;
  const int rotate = !(flags & TFP8_REF_NO_ROTATION);
  const double Q = code_qmax(flags);
  const double rootB = sqrt((double)block);
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int64_t k = 0; k < nb; ++k) {
    /* w = H z with H unnormalised: H x_hat = sqrt(B) (s/alpha) dec(q) because (H/sqrt(B))^2 = I;
       without the rotation, w = z = (s/alpha) dec(q) + g. */
    double *w = (double *)malloc(sizeof(double) * (size_t)block);
    for (int i = 0; i < block; ++i) w[i] = load_elem(grad, grad_dtype, k * block + i);
    if (rotate) tfp8_ref_fwht(w, block);
    double g = (scale[k] == 0.0f) ? 0.0 : (double)scale[k] / (double)alpha[k];
    if (rotate) g *= rootB;
    for (int i = 0; i < block; ++i) w[i] += g * code_value(codes[k * block + i], flags);
    /* energy: sum(z^2) = sum(w^2) / B with the rotation (Parseval), sum(w^2) without */
    double aw = 0.0, sumsq = 0.0;
    for (int i = 0; i < block; ++i) {
      aw = fmax(aw, fabs(w[i]));
      sumsq += w[i] * w[i];
    }
    uint8_t *qo = codes_out + k * block;
    if (aw == 0.0) {
      alpha_out[k] = 1.0f;
      scale_out[k] = 0.0f;
      for (int i = 0; i < block; ++i) {
        qo[i] = 0x00;
        if (quot) quot[k * block + i] = 0.0;
      }
      free(w);
      continue;
    }
    double m2 = (rotate ? sumsq / block : sumsq) / block;
    double a = sqrt((double)target / m2);
    a = fmin(fmax(a, 0x1p-126), 0x1p126);
    float alpha2 = (float)a;
    /* y = alpha H z / sqrt(B) = alpha w / sqrt(B) (rotated), alpha z (not rotated) */
    double div = rotate ? rootB : 1.0;
    float s2 = (float)((double)alpha2 * aw / div / Q);
    for (int i = 0; i < block; ++i) {
      double t = (double)alpha2 * w[i] / div / (double)s2;
      if (quot) quot[k * block + i] = t;
      qo[i] = code_encode(t, flags);
    }
    alpha_out[k] = alpha2;
    scale_out[k] = s2;
    free(w);
  }
  return TFP8_REF_OK;
}
