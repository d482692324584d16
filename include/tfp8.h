/*
 * tfp8.h - C ABI of the MI355X (gfx950) FP8 ASH + DS compression library.
 *
 * Four operations on flat buffers in device memory, each launched asynchronously on the
 * caller's HIP stream:
 *
 *   tfp8_compress    per block of `block` elements: second moment, adaptive prescale alpha_k
 *                    that brings that energy to `target`, orthogonal Hadamard rotation,
 *                    post-scale s_k = max|y| / 448, FP8 E4M3FN codes.  Page "TACO: Efficient
 *                    Communication Compression of Intermediate Tensors for Scalable
 *                    Tensor-Parallel LLM Training", sections 2.A (E4M3), 2.B.1 (adaptive
 *                    scale-Hadamard transform), 2.B.2 (dual-scale quantization) and 2.B.3 (one
 *                    fused kernel for the energy, the transform and the quantization).
 *   tfp8_decompress  the inverse with both scales (same page, section 2.B.2, reconstruction).
 *   tfp8_reduce_fp8  the local step of a two-shot all-reduce: dequantize P contributions,
 *                    sum them, requantize to the same format.  Page "AGoQ: Activation and
 *                    Gradient Quantization for Memory-Efficient Distributed Training of LLMs",
 *                    section 2.B (precision-preserving all-reduce); the TACO page, section
 *                    2.B.3, puts the same step between ReduceScatter and AllGather.
 *   tfp8_accumulate  a compressed main gradient plus a dense local gradient, requantized (the
 *                    AGoQ page, section 2.B, local accumulation); declared at the end.
 *
 * Definitions (readings of the pages; B = block, T = target, Q = 448):
 *   block k covers x[kB, (k+1)B) of the flat row-major buffer; H is the Sylvester Hadamard
 *   matrix of order B in natural order, H[i][j] = (-1)^popcount(i & j), used as H / sqrt(B);
 *   m2 = mean(v^2);  alpha = clamp(sqrt(T / m2), 2^-126, 2^126);  y = H (alpha v) / sqrt(B);
 *   s = max|y| / Q;  code_i = E4M3FN(y_i / s), round to nearest even.  A block whose elements
 *   are all zero stores alpha = 1, s = 0 and codes 0x00, and reconstructs to +0.
 *   Reconstruction: xhat = H (s dec(code)) / (sqrt(B) alpha).
 *   Reduce: z = sum_p xhat_p, then compress z with the same B and T.
 *
 * Conventions shared by all entry points:
 *   - Every data pointer is a DEVICE pointer; `stream` is a hipStream_t (NULL = default stream).
 *   - The caller owns every buffer.  The library allocates and frees nothing and never
 *     synchronizes; outputs are complete when the stream reaches the launch.
 *   - Element counts are 64-bit, at most TFP8_MAX_N (2^40, several times any one GPU's
 *     memory, so that no byte count or address computed from n can overflow).  n = 0 is a
 *     no-op: once block, n, the data type, target, flags, P and the strides pass their checks
 *     the call returns TFP8_OK, and no pointer is examined (NULL, misaligned or overlapping
 *     pointers are accepted).
 *   - Supported block sizes: 64, 128, 256, 512.
 *   - Alignment: x, out and every codes pointer 16 bytes; alpha and scale 4 bytes.
 *   - Out-of-place (except tfp8_accumulate, which may work in place): an output range that
 *     overlaps an input range, or another output range, is rejected with TFP8_E_ARG.
 *   - target must be finite and within [2^-64, 2^64].
 *   - Inputs must be finite with |x| < 2^100; other values are outside the contract (no
 *     check, unspecified codes).
 *   - Argument errors return before any HIP call and nothing is launched.  A launch failure
 *     returns TFP8_E_HIP.  Faults during execution surface at the caller's next
 *     synchronization, as for any HIP kernel.
 *   - Every entry point may be called from several host threads at once: the library keeps no
 *     state beyond a per-device count of compute units, looked up once.  Work launched on the
 *     same buffers from different streams is ordered only by the caller.
 *   - Launches go to the current HIP device; the pointers must belong to it.
 */
#ifndef TFP8_H
#define TFP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TFP8_OK = 0,
  TFP8_E_NULL = -1,  /* a required pointer is NULL (n > 0) */
  TFP8_E_SIZE = -2,  /* n < 0, n > TFP8_MAX_N, or n is not a multiple of block */
  TFP8_E_BLOCK = -3, /* block is not one of 64, 128, 256, 512 */
  TFP8_E_DTYPE = -4, /* dtype is not TFP8_BF16 or TFP8_F32 */
  TFP8_E_ALIGN = -5, /* a pointer is not aligned as stated above */
  TFP8_E_ARG = -6,   /* P < 1 or P > 64, bad target, unknown flags, or overlapping buffers */
  TFP8_E_HIP = -7    /* the HIP runtime rejected the launch */
} tfp8_status;

typedef enum { TFP8_BF16 = 0, TFP8_F32 = 1 } tfp8_dtype;

#define TFP8_MAX_N ((int64_t)1 << 40)

/* Variant flags of the *_ex entry points (0 = the method as defined above):
 *   TFP8_FLAG_INT8         codes are int8 (two's complement, round to nearest even, saturating at
 *                          +-127) with Q_max = 127 instead of E4M3 with 448: the INT8 fallback the
 *                          TACO page keeps for hardware without FP8 (section 5).  Compress,
 *                          decompress and reduce must be called with the same flags.
 *   TFP8_FLAG_NO_ROTATION  leave the Hadamard rotation out (H = identity): plain per-block
 *                          dual-scale quantization, for ablations of the transform. */
#define TFP8_FLAG_INT8 1u
#define TFP8_FLAG_NO_ROTATION 2u
#define TFP8_FLAGS_ALL (TFP8_FLAG_INT8 | TFP8_FLAG_NO_ROTATION)

/* Compress x[n] (bfloat16 or float32, row-major flat) in blocks of `block`.
 * Outputs: codes[n] (E4M3FN bytes, same element order as x), alpha[n/block], scale[n/block]
 * (float32 per block: the prescale alpha_k and the post-scale s_k). */
tfp8_status tfp8_compress(const void *x, tfp8_dtype x_dtype, int64_t n, int32_t block, float target,
                          uint8_t *codes, float *alpha, float *scale, void *stream);

/* Reconstruct out[n] (float32 or bfloat16, rounded to nearest even) from codes[n] and the
 * per-block alpha[n/block], scale[n/block] written by tfp8_compress or tfp8_reduce_fp8. */
tfp8_status tfp8_decompress(const uint8_t *codes, const float *alpha, const float *scale, int64_t n,
                            int32_t block, void *out, tfp8_dtype out_dtype, void *stream);

/* Local reduce of P contributions of the same n elements, stacked contiguously:
 * codes[P][n], alpha[P][n/block], scale[P][n/block] (contribution p at offset p*n, p*n/block).
 * The contributions are dequantized and summed in the order p = 0..P-1 in float64 (at least as
 * precise as the FP32 sum of the AGoQ page), and the sum is requantized with the same block and
 * target into codes_out[n], alpha_out[n/block], scale_out[n/block].  1 <= P <= 64.
 * Precision: each element of the sum (in the rotated domain, r = sum_p (s_p / alpha_p) dec(q_p))
 * is within 2^-44 of the sum of its terms' magnitudes.  Contributions that cancel down to about
 * 2^-25 of their peaks requantize like the exact sum; a contribution and its exact negation give
 * exactly zero when no smaller contribution lies between them in the order.  Where a block's
 * contributions cancel to far below their peaks, its requantized codes carry the float64 sum's
 * rounding noise, as any float64 evaluation of the sum would. */
tfp8_status tfp8_reduce_fp8(const uint8_t *codes, const float *alpha, const float *scale, int32_t P,
                            int64_t n, int32_t block, float target, uint8_t *codes_out,
                            float *alpha_out, float *scale_out, void *stream);

/* The same three operations with variant flags (TFP8_FLAG_*); unknown bits give TFP8_E_ARG.
 * tfp8_compress, tfp8_decompress and tfp8_reduce_fp8 are these with flags = 0.  The reduce only
 * needs the code format: its result is the same with or without the rotation. */
tfp8_status tfp8_compress_ex(const void *x, tfp8_dtype x_dtype, int64_t n, int32_t block,
                             float target, uint32_t flags, uint8_t *codes, float *alpha,
                             float *scale, void *stream);
tfp8_status tfp8_decompress_ex(const uint8_t *codes, const float *alpha, const float *scale,
                               int64_t n, int32_t block, uint32_t flags, void *out,
                               tfp8_dtype out_dtype, void *stream);
tfp8_status tfp8_reduce_ex(const uint8_t *codes, const float *alpha, const float *scale, int32_t P,
                           int64_t n, int32_t block, float target, uint32_t flags,
                           uint8_t *codes_out, float *alpha_out, float *scale_out, void *stream);

/* The local reduce with the P contributions at caller-chosen strides, so that it can read them
 * where a collective left them: for example a receive buffer holding one message per peer,
 * [codes | alpha | scale] back to back, which one all-to-all can fill.  Contribution p is
 *   codes + p * codes_stride  (bytes),  alpha + p * alpha_stride,  scale + p * scale_stride
 * (floats), each n codes or n/block scales long.  codes_stride >= n and a multiple of 16;
 * alpha_stride, scale_stride >= n/block; all strides <= TFP8_MAX_N (TFP8_E_SIZE above it,
 * TFP8_E_ARG below the row length, TFP8_E_ALIGN for codes_stride % 16 != 0).  The inputs may
 * overlap one another (they are only read).  Each input's span runs from its pointer to the end
 * of its last contribution; an output that overlaps any input span, or another output, is
 * TFP8_E_ARG.  The result is that of tfp8_reduce_ex on the same contributions stacked
 * contiguously, bit for bit; tfp8_reduce_ex is this call with codes_stride = n and
 * alpha_stride = scale_stride = n/block.  Same pages as tfp8_reduce_fp8 (the AGoQ page,
 * section 2.B, reduces chunks received from the other ranks). */
tfp8_status tfp8_reduce_strided(const uint8_t *codes, int64_t codes_stride, const float *alpha,
                                int64_t alpha_stride, const float *scale, int64_t scale_stride,
                                int32_t P, int64_t n, int32_t block, float target, uint32_t flags,
                                uint8_t *codes_out, float *alpha_out, float *scale_out,
                                void *stream);

/* Local gradient accumulation: the compressed main gradient (codes[n], alpha[n/block],
 * scale[n/block], as written by tfp8_compress_ex with the same flags) is dequantized, the dense
 * local gradient grad[n] (bfloat16 or float32) is added, and the sum is requantized with the same
 * block, target and flags into codes_out, alpha_out, scale_out.  Page "AGoQ: Activation and
 * Gradient Quantization for Memory-Efficient Distributed Training of LLMs", section 2.B (local
 * accumulation of FP8 gradients across micro-batches).  The sum is formed in float32 (the page
 * names FP16/BF16 as its minimum precision); blocks where the two terms cancel to under half of
 * the larger one are redone by a second kernel that forms the sum in float64 with the roundings of
 * the definition (reconstruction, then + grad), so that terms which cancel exactly give exactly
 * zero and every later error is relative to the sum.  Unlike the other calls this one may work
 * in place: each of codes_out, alpha_out, scale_out may be exactly its input (any other overlap
 * is TFP8_E_ARG).  grad must be 16-byte aligned. */
tfp8_status tfp8_accumulate(const uint8_t *codes, const float *alpha, const float *scale,
                            const void *grad, tfp8_dtype grad_dtype, int64_t n, int32_t block,
                            float target, uint32_t flags, uint8_t *codes_out, float *alpha_out,
                            float *scale_out, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *tfp8_status_string(tfp8_status status);

/* ABI version of this header: (major << 16) | minor. */
int32_t tfp8_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TFP8_H */
