/*
 * tfp8_c_driver.c - drives libtfp8.so from plain C99 through include/tfp8.h, with no Python and
 * no torch: the C ABI as a C caller sees it.
 *
 *   tfp8_c_driver errors
 *       Calls every entry point with arguments the header documents as errors and checks the
 *       returned status.  These paths return before any HIP call, so this mode needs no GPU.
 *
 *   tfp8_c_driver compress   <dir> <n> <block> <target>
 *   tfp8_c_driver reduce     <dir> <n> <block> <target> <P>
 *   tfp8_c_driver decompress <dir> <n> <block>
 *       One operation on the GPU.  Inputs are read from raw files in <dir>, copied to device
 *       memory taken with hipMalloc, the operation is launched on a stream of its own
 *       (hipStreamCreate), and the outputs are written back to raw files in <dir>:
 *         compress:   x.bf16 (n bfloat16)          -> codes.u8, alpha.f32, scale.f32
 *         reduce:     in_codes.u8 (P n), in_alpha.f32, in_scale.f32 (P n/block each)
 *                                                  -> codes.u8, alpha.f32, scale.f32
 *         decompress: in_codes.u8 (n), in_alpha.f32, in_scale.f32 -> out.f32 (n float32)
 *
 * Prints one line per step and exits 0 on success, 1 on any failure.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tfp8.h"

static int failures = 0;

static void expect(const char *what, tfp8_status got, tfp8_status want) {
  if (got != want) {
    printf("FAIL %s: status %d (%s), expected %d\n", what, (int)got, tfp8_status_string(got),
           (int)want);
    ++failures;
  }
}

/* Host addresses that are 16-byte aligned and never dereferenced: argument checks run first. */
#define FAKE(off) ((void *)((uintptr_t)0x7F0000000000u + (uintptr_t)(off)))

static int run_errors(void) {
  uint8_t *q = (uint8_t *)FAKE(0), *q2 = (uint8_t *)FAKE(1 << 20);
  float *a = (float *)FAKE(2 << 20), *s = (float *)FAKE(3 << 20);
  float *a2 = (float *)FAKE(4 << 20), *s2 = (float *)FAKE(5 << 20);
  const void *x = FAKE(6 << 20);
  void *out = FAKE(8 << 20);

  if ((tfp8_version() >> 16) != 1) {
    printf("FAIL version %d\n", (int)tfp8_version());
    ++failures;
  }
  if (strcmp(tfp8_status_string(TFP8_OK), "ok") != 0) {
    printf("FAIL status string\n");
    ++failures;
  }
  expect("compress block 96", tfp8_compress(x, TFP8_BF16, 1024, 96, 1.0f, q, a, s, NULL),
         TFP8_E_BLOCK);
  expect("compress n % block", tfp8_compress(x, TFP8_BF16, 1000, 128, 1.0f, q, a, s, NULL),
         TFP8_E_SIZE);
  expect("compress n > 2^40",
         tfp8_compress(x, TFP8_BF16, TFP8_MAX_N + 128, 128, 1.0f, q, a, s, NULL), TFP8_E_SIZE);
  expect("compress dtype", tfp8_compress(x, (tfp8_dtype)7, 1024, 128, 1.0f, q, a, s, NULL),
         TFP8_E_DTYPE);
  expect("compress target 0", tfp8_compress(x, TFP8_BF16, 1024, 128, 0.0f, q, a, s, NULL),
         TFP8_E_ARG);
  expect("compress flags", tfp8_compress_ex(x, TFP8_BF16, 1024, 128, 1.0f, 4u, q, a, s, NULL),
         TFP8_E_ARG);
  expect("compress NULL", tfp8_compress(NULL, TFP8_BF16, 1024, 128, 1.0f, q, a, s, NULL),
         TFP8_E_NULL);
  expect("compress misaligned x",
         tfp8_compress((const char *)x + 2, TFP8_BF16, 1024, 128, 1.0f, q, a, s, NULL),
         TFP8_E_ALIGN);
  expect("compress overlap", tfp8_compress(x, TFP8_BF16, 1024, 128, 1.0f, q, a, a, NULL),
         TFP8_E_ARG);
  expect("compress n = 0", tfp8_compress(NULL, TFP8_BF16, 0, 128, 1.0f, NULL, NULL, NULL, NULL),
         TFP8_OK);
  expect("decompress n < 0", tfp8_decompress(q, a, s, -128, 128, out, TFP8_F32, NULL),
         TFP8_E_SIZE);
  expect("decompress dtype", tfp8_decompress(q, a, s, 1024, 128, out, (tfp8_dtype)2, NULL),
         TFP8_E_DTYPE);
  expect("decompress overlap", tfp8_decompress(q, a, s, 1024, 128, (void *)q, TFP8_F32, NULL),
         TFP8_E_ARG);
  expect("reduce P = 0", tfp8_reduce_fp8(q, a, s, 0, 1024, 128, 1.0f, q2, a2, s2, NULL),
         TFP8_E_ARG);
  expect("reduce P = 65", tfp8_reduce_fp8(q, a, s, 65, 1024, 128, 1.0f, q2, a2, s2, NULL),
         TFP8_E_ARG);
  expect("reduce in place", tfp8_reduce_fp8(q, a, s, 2, 1024, 128, 1.0f, q, a2, s2, NULL),
         TFP8_E_ARG);
  expect("reduce_ex flags", tfp8_reduce_ex(q, a, s, 2, 1024, 128, 1.0f, 8u, q2, a2, s2, NULL),
         TFP8_E_ARG);
  expect("reduce_strided stride below n",
         tfp8_reduce_strided(q, 1008, a, 8, s, 8, 2, 1024, 128, 1.0f, 0u, q2, a2, s2, NULL),
         TFP8_E_ARG);
  expect("reduce_strided stride % 16",
         tfp8_reduce_strided(q, 1032, a, 8, s, 8, 2, 1024, 128, 1.0f, 0u, q2, a2, s2, NULL),
         TFP8_E_ALIGN);
  expect("accumulate NULL grad",
         tfp8_accumulate(q, a, s, NULL, TFP8_BF16, 1024, 128, 1.0f, 0u, q, a, s, NULL),
         TFP8_E_NULL);
  expect("accumulate partial overlap",
         tfp8_accumulate(q, a, s, x, TFP8_BF16, 1024, 128, 1.0f, 0u, q + 16, a, s, NULL),
         TFP8_E_ARG);
  printf("errors: %s\n", failures ? "FAILED" : "ok");
  return failures ? 1 : 0;
}

/* ---------------------------------------------------------------------------- GPU operations */

static void *read_file(const char *dir, const char *name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) {
    printf("FAIL cannot open %s\n", path);
    return NULL;
  }
  void *buf = malloc(bytes ? bytes : 1);
  const size_t got = buf ? fread(buf, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    printf("FAIL %s: read %zu of %zu bytes\n", path, got, bytes);
    free(buf);
    return NULL;
  }
  return buf;
}

static int write_file(const char *dir, const char *name, const void *buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f) return 1;
  const size_t put = fwrite(buf, 1, bytes, f);
  return (fclose(f) != 0 || put != bytes) ? 1 : 0;
}

#define HIP_OK(call)                                                               \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) {                                                        \
      printf("FAIL %s: %s\n", #call, hipGetErrorString(e_));                       \
      return 1;                                                                    \
    }                                                                              \
  } while (0)

/* Copies `bytes` from host `src` to a new device buffer. */
static int to_device(void **dev, const void *src, size_t bytes) {
  HIP_OK(hipMalloc(dev, bytes));
  HIP_OK(hipMemcpy(*dev, src, bytes, hipMemcpyHostToDevice));
  return 0;
}

static int from_device(const char *dir, const char *name, const void *dev, size_t bytes) {
  void *host = malloc(bytes);
  if (!host) return 1;
  const hipError_t e = hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost);
  const int bad = (e != hipSuccess) || write_file(dir, name, host, bytes);
  if (bad) printf("FAIL writing %s\n", name);
  free(host);
  return bad;
}

static int run_gpu(const char *op, const char *dir, int64_t n, int32_t block, float target,
                   int32_t P) {
  const int64_t nb = n / block;
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  tfp8_status status = TFP8_OK;
  void *d_in = NULL, *d_a = NULL, *d_s = NULL, *d_q = NULL, *d_oa = NULL, *d_os = NULL,
       *d_out = NULL;
  int bad = 0;

  if (strcmp(op, "compress") == 0) {
    void *x = read_file(dir, "x.bf16", (size_t)n * 2);
    if (!x) return 1;
    bad |= to_device(&d_in, x, (size_t)n * 2);
    free(x);
    HIP_OK(hipMalloc(&d_q, (size_t)n));
    HIP_OK(hipMalloc(&d_oa, (size_t)nb * 4));
    HIP_OK(hipMalloc(&d_os, (size_t)nb * 4));
    if (!bad)
      status = tfp8_compress(d_in, TFP8_BF16, n, block, target, (uint8_t *)d_q, (float *)d_oa,
                             (float *)d_os, (void *)st);
  } else if (strcmp(op, "reduce") == 0 || strcmp(op, "decompress") == 0) {
    const int is_reduce = strcmp(op, "reduce") == 0;
    const int64_t parts = is_reduce ? P : 1;
    void *q = read_file(dir, "in_codes.u8", (size_t)(parts * n));
    void *a = read_file(dir, "in_alpha.f32", (size_t)(parts * nb) * 4);
    void *s = read_file(dir, "in_scale.f32", (size_t)(parts * nb) * 4);
    if (!q || !a || !s) return 1;
    bad |= to_device(&d_in, q, (size_t)(parts * n));
    bad |= to_device(&d_a, a, (size_t)(parts * nb) * 4);
    bad |= to_device(&d_s, s, (size_t)(parts * nb) * 4);
    free(q);
    free(a);
    free(s);
    if (is_reduce) {
      HIP_OK(hipMalloc(&d_q, (size_t)n));
      HIP_OK(hipMalloc(&d_oa, (size_t)nb * 4));
      HIP_OK(hipMalloc(&d_os, (size_t)nb * 4));
      if (!bad)
        status = tfp8_reduce_fp8((const uint8_t *)d_in, (const float *)d_a, (const float *)d_s,
                                 P, n, block, target, (uint8_t *)d_q, (float *)d_oa,
                                 (float *)d_os, (void *)st);
    } else {
      HIP_OK(hipMalloc(&d_out, (size_t)n * 4));
      if (!bad)
        status = tfp8_decompress((const uint8_t *)d_in, (const float *)d_a, (const float *)d_s,
                                 n, block, d_out, TFP8_F32, (void *)st);
    }
  } else {
    printf("FAIL unknown operation %s\n", op);
    return 1;
  }
  if (bad) return 1;
  if (status != TFP8_OK) {
    printf("FAIL %s: %s\n", op, tfp8_status_string(status));
    return 1;
  }
  HIP_OK(hipStreamSynchronize(st));
  if (d_out) {
    bad |= from_device(dir, "out.f32", d_out, (size_t)n * 4);
  } else {
    bad |= from_device(dir, "codes.u8", d_q, (size_t)n);
    bad |= from_device(dir, "alpha.f32", d_oa, (size_t)nb * 4);
    bad |= from_device(dir, "scale.f32", d_os, (size_t)nb * 4);
  }
  hipFree(d_in);
  hipFree(d_a);
  hipFree(d_s);
  hipFree(d_q);
  hipFree(d_oa);
  hipFree(d_os);
  hipFree(d_out);
  HIP_OK(hipStreamDestroy(st));
  printf("%s: n=%lld block=%d%s\n", op, (long long)n, (int)block, bad ? " FAILED" : " ok");
  return bad;
}

int main(int argc, char **argv) {
  if (argc >= 2 && strcmp(argv[1], "errors") == 0) return run_errors();
  if (argc >= 5) {
    const int64_t n = strtoll(argv[3], NULL, 10);
    const int32_t block = (int32_t)strtol(argv[4], NULL, 10);
    const float target = argc >= 6 ? strtof(argv[5], NULL) : 1.0f;
    const int32_t P = argc >= 7 ? (int32_t)strtol(argv[6], NULL, 10) : 1;
    if (n <= 0 || block <= 0 || n % block != 0 || P < 1) {
      printf("FAIL bad sizes\n");
      return 1;
    }
    return run_gpu(argv[1], argv[2], n, block, target, P);
  }
  fprintf(stderr,
          "usage: %s errors | compress DIR N BLOCK TARGET | reduce DIR N BLOCK TARGET P | "
          "decompress DIR N BLOCK\n",
          argv[0]);
  return 2;
}
