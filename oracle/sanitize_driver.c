/*
 * sanitize_driver.c -- test infrastructure only: drives every entry point of
 * razer_oracle.c over ordinary, edge-case and rejected inputs so that a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py)
 * sees every loop bound and table index the oracle uses.  Exit status 0 and
 * no sanitizer report means clean; a wrong status from an argument check
 * exits 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "razer_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static double uniform(void) {
  /* splitmix64 -> [0, 1) */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}

static float normal(void) {
  double u1 = uniform(), u2 = uniform();
  if (u1 < 1e-300) u1 = 1e-300;
  return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

static int fail(const char* what) {
  fprintf(stderr, "sanitize_driver: %s\n", what);
  return 1;
}

/* One tensor through every mode, block size and scale format it allows, then
 * dequant and the product over all rows and over a column subset. */
static int run_tensor(const float* x, int64_t rows, int64_t cols) {
  static const int blocks[4] = {16, 32, 64, 128};
  int8_t off_w[2] = {-2, -5}, off_a[2] = {-2, 0};
  for (int kind = 0; kind < 2; kind++) {
    const int8_t* off = kind == RZO_WEIGHT ? off_w : off_a;
    for (int bi = 0; bi < 4; bi++) {
      const int block = blocks[bi];
      if (cols % block) continue;
      for (int sfmt = 0; sfmt < (kind == RZO_WEIGHT ? 2 : 1); sfmt++) {
        for (int mode = 0; mode < 3; mode++) {
          const int64_t n = rows * cols;
          uint8_t* codes = malloc((size_t)(n / 2 + 1));
          void* scales = malloc((size_t)(n / block * (sfmt ? 2 : 1) + 1));
          float ts = 0.0f;
          if (rzo_quantize_fmt(kind, x, rows, cols, off, mode, block, sfmt, codes, scales, &ts) != 0)
            return fail("quantize_fmt rejected valid arguments");
          double* d64 = malloc((size_t)(n + 1) * sizeof(double));
          float* d32 = malloc((size_t)(n + 1) * sizeof(float));
          rzo_dequant_fmt_f64(kind, block, sfmt, codes, scales, ts, off, rows, cols, d64);
          rzo_dequant_fmt_f32(kind, block, sfmt, codes, scales, ts, off, rows, cols, d32);
          if (block == 16 && sfmt == 0) {
            float* xv = malloc((size_t)(2 * cols + 1) * sizeof(float));
            for (int64_t k = 0; k < 2 * cols; k++) xv[k] = normal();
            double* y = malloc((size_t)(2 * (rows > 3 ? rows : 3) + 1) * sizeof(double));
            double* nrm = malloc((size_t)(2 * (rows > 3 ? rows : 3) + 1) * sizeof(double));
            rzo_gemm(xv, 2, cols, kind, codes, scales, ts, off, rows, NULL, rows, y, nrm);
            int64_t idx[3] = {rows - 1, 0, rows / 2};
            rzo_gemm(xv, 2, cols, kind, codes, scales, ts, off, rows, idx, 3, y, nrm);
            rzo_dequant_f64(kind, codes, scales, ts, off, rows, cols, d64);
            rzo_dequant_f32(kind, codes, scales, ts, off, rows, cols, d32);
            uint8_t* c2 = malloc((size_t)(n / 2 + 1));
            uint8_t* s2 = malloc((size_t)(n / 16 + 1));
            if (rzo_quantize(kind, x, rows, cols, off, mode, c2, s2, &ts) != 0)
              return fail("quantize rejected valid arguments");
            free(xv); free(y); free(nrm); free(c2); free(s2);
          }
          free(codes); free(scales); free(d64); free(d32);
        }
      }
    }
  }
  return 0;
}

int main(void) {
  /* scalar helpers over their whole domains */
  for (int c = 0; c < 16; c++) (void)rzo_fp4_value(c);
  for (int i = -4; i < 200; i++) (void)rzo_fp4_round_mag(i * 0.0625);
  (void)rzo_fp4_round_mag(1e30);
  for (int kind = 0; kind < 2; kind++) {
    for (int c = 0; c < 128; c++) (void)rzo_scale_value(kind, c);
    for (int c = 0; c < 256; c++) {
      (void)rzo_block_scale(kind, c);
      int8_t off[2] = {-7, 7};
      for (int code = 0; code < 16; code++) (void)rzo_decode_value(kind, code, c, off);
    }
    const float probes[] = {0.0f, 1e-30f, 0.001f, 0.5f, 1.0f, 29.9f, 30.0f, 31.0f, 447.0f, 448.0f,
                            500.0f, 1e30f, INFINITY};
    for (size_t i = 0; i < sizeof probes / sizeof probes[0]; i++) {
      (void)rzo_scale_round(kind, probes[i]);
      (void)rzo_scale_round_fmt(kind, RZO_SCALE_BYTE, probes[i]);
      if (kind == RZO_WEIGHT) (void)rzo_scale_round_fmt(kind, RZO_SCALE_F16, probes[i]);
    }
    (void)rzo_scale_max(kind);
    (void)rzo_scale_max_fmt(kind, RZO_SCALE_BYTE);
  }
  for (int c = 0; c < 0x4000; c += 7) (void)rzo_scale_value_fmt(RZO_WEIGHT, RZO_SCALE_F16, c);
  for (int o = -7; o <= 7; o++) (void)rzo_special_value(o & 1, o);

  /* block remap at every block length with 4 candidates */
  {
    float y[128];
    uint8_t codes[128];
    double cand[4] = {5.0, -5.0, 3.5, -3.5};
    for (int n = 1; n <= 128; n++) {
      for (int j = 0; j < n; j++) y[j] = 3.0f * normal();
      int sel = -1;
      rzo_encode_block_scaled(y, n, cand, 4, 1, codes, &sel);
      if (sel < 0 || sel > 3) return fail("selection out of range");
      rzo_encode_block_scaled(y, n, cand, 4, 0, codes, &sel);
    }
  }

  /* tensors: ordinary, ragged, outliers, zeros, subnormals, non-finite */
  const int64_t rows = 5, cols = 256;
  float* x = malloc((size_t)(rows * cols) * sizeof(float));
  for (int64_t i = 0; i < rows * cols; i++) x[i] = 0.02f * normal();
  x[17] = 3.0f;
  if (run_tensor(x, rows, cols)) return 1;
  if (run_tensor(x, 3, 48)) return 1;
  if (run_tensor(x, 1, 16)) return 1;
  memset(x, 0, (size_t)(rows * cols) * sizeof(float));
  if (run_tensor(x, rows, cols)) return 1;
  for (int64_t i = 0; i < rows * cols; i++) x[i] = 1e-40f * (float)(i % 7);
  x[3] = 1.0f;
  if (run_tensor(x, rows, cols)) return 1;
  x[40] = NAN;
  if (run_tensor(x, rows, cols)) return 1;
  x[40] = -INFINITY;
  if (run_tensor(x, rows, cols)) return 1;
  if (run_tensor(x, 0, cols)) return 1;

  /* rejected arguments write nothing and return -1 */
  {
    uint8_t codes[8], scales[8];
    float ts = 0.0f;
    int8_t off[2] = {-2, 4}, bad[2] = {-2, 9};
    if (rzo_quantize(RZO_WEIGHT, x, 1, 15, off, RZO_MODE_RAZER, codes, scales, &ts) != -1)
      return fail("cols % 16 accepted");
    if (rzo_quantize(RZO_WEIGHT, x, 1, 16, bad, RZO_MODE_RAZER, codes, scales, &ts) != -1)
      return fail("offset 9 accepted");
    if (rzo_quantize(7, x, 1, 16, off, RZO_MODE_RAZER, codes, scales, &ts) != -1)
      return fail("kind 7 accepted");
    if (rzo_quantize_fmt(RZO_WEIGHT, x, 1, 16, off, RZO_MODE_RAZER, 8, 0, codes, scales, &ts) != -1)
      return fail("block 8 accepted");
    if (rzo_quantize_fmt(RZO_ACT, x, 1, 16, off, RZO_MODE_RAZER, 16, RZO_SCALE_F16, codes, scales, &ts) != -1)
      return fail("FP16 scales for activations accepted");
    if (rzo_quantize(RZO_WEIGHT, x, -1, 16, off, RZO_MODE_RAZER, codes, scales, &ts) != -1)
      return fail("negative rows accepted");
  }
  free(x);
  printf("sanitize_driver: ok\n");
  return 0;
}
