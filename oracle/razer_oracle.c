/*
 * razer_oracle.c -- CPU oracle for RaZeR-NVFP4 (test infrastructure only).
 *
 * Only the tests, the smoke check and the bench's CPU-baseline leg load this
 * file's library.  It is deliberately plain: linear scans instead of bit
 * tricks, fp64 wherever a value is compared, one element at a time, one thread.
 * See razer_oracle.h for the page names abbreviated [notes] and [summary].
 *
 * Readings of points the pages leave open (each is listed with its reason in
 * the design notes of the repository):
 *   - tensor scale st = amax_tensor / (6 * S_MAX); block scale code =
 *     nearest(S_MAX * amax_block / amax_tensor)   ([notes] Background: the
 *     FP8 block scale is the block absolute max divided by a global maximum)
 *   - E3M3 = 3 exponent bits with bias 3, 3 mantissa bits, subnormals, no
 *     Inf/NaN (max 30); E4M3 = OCP E4M3FN (max 448)
 *   - every rounding is to nearest, ties to the even code; scale codes
 *     saturate at the format maximum; FP4 saturates at 6
 *   - an element takes the special value only if it is strictly closer to it
 *     than to its FP4 rounding (a tie keeps the regular FP4 value)
 *   - candidate ties go to the lowest candidate index (+M0, -M0, +M1, -M1)
 *   - metadata: bit 7 = sign of the special value, bit 6 = pair (weights)
 *   - fp32 op order: r = amax_b / amax_t; sb_real = r * S_MAX; D = sb * st;
 *     R = 1 / D; y = x * R (no fused multiply-add anywhere; build with
 *     -ffp-contract=off)
 *   - Four Over Six baseline: the same tensor scale; per block the second
 *     candidate scale is the nearest code to sb_real * 1.5 (max -> 4,
 *     saturating like any scale code); both candidates are plain FP4 and the
 *     block keeps the one with the smaller fp64 squared error in real units,
 *     a tie keeping max -> 6
 */
#include "razer_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* FP4-E2M1 magnitudes by 3-bit magnitude field.  [notes] Key design 2 and
 * [summary] §1 list the representable set {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a
 * separate sign bit (sign-magnitude, hence both +0 and -0). */
static const double kFp4Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double rzo_fp4_value(int code) {
  double m = kFp4Mag[code & 7];
  return (code & 8) ? -m : m; /* code 8 gives -0.0: the redundant zero */
}

int rzo_fp4_round_mag(double a) {
  /* Nearest grid magnitude by linear scan.  Only neighbours can tie; on a tie
   * the even index wins (round to nearest even mantissa).  Values at or above
   * 6 saturate to 6 (stated first: for huge a the fp64 distances would tie). */
  if (a >= 6.0) return 7;
  int best = 0;
  double bd = fabs(a - kFp4Mag[0]);
  for (int i = 1; i < 8; i++) {
    double d = fabs(a - kFp4Mag[i]);
    if (d < bd || (d == bd && (i & 1) == 0)) {
      best = i;
      bd = d;
    }
  }
  return best;
}

/* Block-scale formats.  [notes] Key design 1 / [summary] §2.1: activations keep
 * the 8-bit E4M3 scale whose sign bit is free (1 metadata bit); weights trim
 * it to 6-bit E3M3, freeing the sign bit and the top exponent bit (2 bits). */
static double e3m3_value(int code) {
  int e = (code >> 3) & 7, m = code & 7;
  return e == 0 ? ldexp((double)m, -5) : ldexp((double)(8 + m), e - 6);
}

static double e4m3_value(int code) {
  int e = (code >> 3) & 15, m = code & 7;
  return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

double rzo_scale_value(int kind, int code) {
  return kind == RZO_WEIGHT ? e3m3_value(code & 63) : e4m3_value(code & 127);
}

double rzo_scale_max(int kind) { return kind == RZO_WEIGHT ? 30.0 : 448.0; }

int rzo_scale_round(int kind, float v) {
  /* Codes are monotone in value, so the nearest code is found by a scan; the
   * E4M3 NaN code 0x7F is never a candidate.  At or above the maximum the
   * result saturates to the largest code. */
  int ncode = kind == RZO_WEIGHT ? 64 : 127;
  if ((double)v >= rzo_scale_max(kind)) return ncode - 1;
  int best = 0;
  double bd = fabs((double)v - rzo_scale_value(kind, 0));
  for (int c = 1; c < ncode; c++) {
    double d = fabs((double)v - rzo_scale_value(kind, c));
    if (d < bd || (d == bd && (c & 1) == 0)) {
      best = c;
      bd = d;
    }
  }
  return best;
}

/* Group-scale variant: an FP16 block scale whose sign bit and top exponent
 * bit hold the metadata ([notes] Key design 3: the Blackwell kernels use block
 * size 128 and store the metadata in those two bits of the FP16 scale).  The
 * scale itself is the 14-bit remainder: an FP16 number with exponent field
 * 0..15, so values from 2^-24 (subnormal) up to 2 - 2^-10. */
static double f16s_value(int code) {
  int e = (code >> 10) & 15, m = code & 1023;
  return e == 0 ? ldexp((double)m, -24) : ldexp((double)(1024 + m), e - 25);
}

static double f16s_max(void) { return f16s_value(0x3FFF); }

static int f16s_round(float v) {
  /* nearest of the 16384 codes (values increase with the code): the largest
   * code at or below v by bisection, then the nearer of it and the next code,
   * ties to the even code; saturating at the largest code */
  if ((double)v >= f16s_max()) return 0x3FFF;
  int lo = 0, hi = 0x3FFF; /* value(lo) <= v < value(hi) */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (f16s_value(mid) <= (double)v)
      lo = mid;
    else
      hi = mid;
  }
  double dlo = (double)v - f16s_value(lo), dhi = f16s_value(hi) - (double)v;
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo & 1) == 0 ? lo : hi;
}

double rzo_scale_value_fmt(int kind, int sfmt, int code) {
  return sfmt == RZO_SCALE_F16 ? f16s_value(code & 0x3FFF) : rzo_scale_value(kind, code);
}

int rzo_scale_round_fmt(int kind, int sfmt, float v) {
  return sfmt == RZO_SCALE_F16 ? f16s_round(v) : rzo_scale_round(kind, v);
}

double rzo_scale_max_fmt(int kind, int sfmt) {
  return sfmt == RZO_SCALE_F16 ? f16s_max() : rzo_scale_max(kind);
}

double rzo_special_value(int neg, int off_half) {
  /* [notes] Key design 3: a 4-bit offset register holds a fixed-point offset
   * in [-3.5, 3.5] with step 0.5; the decoder adds it to the base 6.0 and
   * attaches the sign.  Offsets are carried in units of 0.5. */
  double mag = 6.0 + (double)off_half / 2.0;
  return neg ? -mag : mag;
}

void rzo_encode_block_scaled(const float* y, int n, const double* cand, int ncand, int remap,
                             uint8_t* codes, int* sel_out) {
  /* [notes] Key design 2, block MSE equation: the block's special value is
   * argmin over v in V of || round(X_scaled, Q_fp4 U {v}) - X_scaled ||^2.
   *
   * Rounding to Q_fp4 U {v}: an element goes to v exactly when v is strictly
   * nearer than its FP4 rounding q0; otherwise it keeps q0.  So the squared
   * error with candidate v differs from the plain-FP4 error only at those
   * elements, by (v - y)^2 - (q0 - y)^2 = (v - q0) * (v + q0 - 2y).  The
   * plain-FP4 error is the same for every candidate, so the argmin over the
   * sums of these differences is the argmin of the equation.  In fp64 each
   * difference is exact (v, q0 are multiples of 0.5 below 16; a moved element
   * has |y| > 2 so y is a multiple of 2^-22 and |y| stays below 2^4), so the
   * sums are exact and the comparison is exact. */
  double q0[128];
  int m0[128];
  for (int j = 0; j < n; j++) {
    double yj = (double)y[j];
    m0[j] = rzo_fp4_round_mag(fabs(yj));
    q0[j] = yj < 0.0 ? -kFp4Mag[m0[j]] : kFp4Mag[m0[j]];
  }
  int sel = 0;
  if (remap) {
    double best = 0.0;
    for (int c = 0; c < ncand; c++) {
      double v = cand[c], delta = 0.0;
      for (int j = 0; j < n; j++) {
        double yj = (double)y[j];
        if (fabs(yj - v) < fabs(yj - q0[j])) delta += (v - q0[j]) * (v + q0[j] - 2.0 * yj);
      }
      if (c == 0 || delta < best) {
        best = delta;
        sel = c;
      }
    }
  }
  for (int j = 0; j < n; j++) {
    double yj = (double)y[j];
    if (remap && fabs(yj - cand[sel]) < fabs(yj - q0[j]))
      codes[j] = 8; /* the redundant -0 slot now means the special value */
    else if (m0[j] == 0)
      codes[j] = 0; /* zero is always written as +0 */
    else
      codes[j] = (uint8_t)((yj < 0.0 ? 8 : 0) | m0[j]);
  }
  *sel_out = sel;
}

static int valid_offsets(int kind, const int8_t* off) {
  int n = kind == RZO_WEIGHT ? 2 : 1;
  for (int i = 0; i < n; i++)
    if (off[i] < -7 || off[i] > 7) return 0;
  return 1;
}

/* One block at real block scale sb_real (in units of the tensor scale): the
 * scale code is the nearest code to sb_real, the elements are divided by the
 * decoded scale times st and rounded (with the special-value search when
 * remap).  Returns the scale code; 0 means the block is stored as zero (the
 * code underflows or the scale product does), and then c16 is all +0. */
static int encode_at_scale(int kind, int sfmt, int n, const float* xb, float sb_real, float st,
                           const double* cand, int ncand, int remap, uint8_t* cb, int* sel) {
  memset(cb, 0, (size_t)n);
  *sel = 0;
  int scode = rzo_scale_round_fmt(kind, sfmt, sb_real);
  if (scode == 0) return 0;
  float sb = (float)rzo_scale_value_fmt(kind, sfmt, scode);
  float d = sb * st;
  float rcp = 1.0f / d;
  if (!isfinite(rcp)) return 0;
  float y[128];
  for (int j = 0; j < n; j++) y[j] = xb[j] * rcp;
  rzo_encode_block_scaled(y, n, cand, ncand, remap, cb, sel);
  return scode;
}

/* Squared error of a plain-FP4 block (no special value) in real units: the
 * sum of (x_j - value_j * sb * st)^2 in fp64, added in element order
 * j = 0 .. n-1.  value * sb * st is exact in fp64 (at most 3 + 11 + 24
 * significant bits); the difference, the square and each partial sum are
 * rounded once each. */
static double block_sse_sv(int kind, int sfmt, int n, const float* xb, const uint8_t* cb, int scode,
                           float st, double sv) {
  double sb = scode == 0 ? 0.0 : rzo_scale_value_fmt(kind, sfmt, scode);
  double sse = 0.0;
  for (int j = 0; j < n; j++) {
    double v = cb[j] == 8 ? sv : rzo_fp4_value(cb[j]);
    double q = v * sb * (double)st;
    double e = (double)xb[j] - q;
    sse += e * e;
  }
  return sse;
}

static double block_sse(int kind, int sfmt, int n, const float* xb, const uint8_t* cb, int scode,
                        float st) {
  /* plain FP4 codes: code 8 never occurs (a negative zero is written +0) */
  return block_sse_sv(kind, sfmt, n, xb, cb, scode, st, 0.0);
}

int rzo_quantize(int kind, const float* x, int64_t rows, int64_t cols, const int8_t* off_half,
                 int mode, uint8_t* codes, uint8_t* scales, float* tensor_scale) {
  return rzo_quantize_fmt(kind, x, rows, cols, off_half, mode, 16, RZO_SCALE_BYTE, codes, scales,
                          tensor_scale);
}

int rzo_quantize_fmt(int kind, const float* x, int64_t rows, int64_t cols, const int8_t* off_half,
                     int mode, int block, int sfmt, uint8_t* codes, void* scales,
                     float* tensor_scale) {
  if ((kind != RZO_WEIGHT && kind != RZO_ACT) || rows < 0 || cols < 0 ||
      (block != 16 && block != 32 && block != 64 && block != 128) || cols % block != 0 ||
      (sfmt != RZO_SCALE_BYTE && sfmt != RZO_SCALE_F16) || (sfmt == RZO_SCALE_F16 && kind != RZO_WEIGHT) ||
      mode < RZO_MODE_PLAIN || mode > RZO_MODE_RAZER_RESCALE ||
      (mode == RZO_MODE_RAZER_RESCALE && (block != 16 || sfmt != RZO_SCALE_BYTE)) ||
      !off_half || !valid_offsets(kind, off_half))
    return -1;
  int64_t n = rows * cols, nblk = n / block;
  const size_t sbytes = sfmt == RZO_SCALE_F16 ? 2 : 1;
  memset(codes, 0, (size_t)(n / 2));
  memset(scales, 0, (size_t)nblk * sbytes);
  if (n == 0) {
    *tensor_scale = 0.0f;
    return 0;
  }

  /* Tensor level: FP32 scale from the tensor's absolute maximum ([notes]
   * Background: NVFP4 pairs the 16-element FP8 block scale with a
   * tensor-level FP32 scale).  Any non-finite input poisons the tensor. */
  float amax = 0.0f;
  int finite = 1;
  for (int64_t i = 0; i < n; i++) {
    if (!isfinite(x[i])) finite = 0;
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  if (!finite) {
    *tensor_scale = NAN;
    return 0;
  }
  if (amax == 0.0f) {
    *tensor_scale = 0.0f;
    return 0;
  }
  const float smax = (float)rzo_scale_max_fmt(kind, sfmt);
  const float st = amax / (6.0f * smax);
  *tensor_scale = st;

  /* Candidate special values, in selection-index order.  Weights: two +/-
   * pairs (2 metadata bits, [notes] Key design 1); activations: one pair
   * (1 bit). */
  double cand[4];
  int ncand;
  if (kind == RZO_WEIGHT) {
    cand[0] = rzo_special_value(0, off_half[0]);
    cand[1] = rzo_special_value(1, off_half[0]);
    cand[2] = rzo_special_value(0, off_half[1]);
    cand[3] = rzo_special_value(1, off_half[1]);
    ncand = 4;
  } else {
    cand[0] = rzo_special_value(0, off_half[0]);
    cand[1] = rzo_special_value(1, off_half[0]);
    ncand = 2;
  }

  for (int64_t b = 0; b < nblk; b++) {
    const float* xb = x + (int64_t)block * b;
    float amax_b = 0.0f;
    for (int j = 0; j < block; j++) {
      float a = fabsf(xb[j]);
      if (a > amax_b) amax_b = a;
    }
    float r = amax_b / amax;
    float sb_real = r * smax;
    uint8_t cb[128];
    int sel = 0;
    int scode = 0;
    if (mode == RZO_MODE_RAZER_RESCALE) {
      /* Rescaled large special values (a reading of [notes] Training
       * strategy, whose best weight pairs include +/-7, +/-8 and +/-9, values
       * a block scaled max -> 6 almost never reaches): candidate c alone, at
       * the block scale that maps the maximum to |v_c| when |v_c| > 6.  The
       * error of each encoding is summed in real units in fp64 in element
       * order (every term value * sb * st exact), and the smallest wins, ties
       * to the lowest index.  A candidate whose scale code or scale product
       * underflows stores the block as zero (error = sum of x^2). */
      double best = 0.0;
      for (int c = 0; c < ncand; c++) {
        double mag = fabs(cand[c]);
        float sbr = mag > 6.0 ? (sb_real * 6.0f) / (float)mag : sb_real;
        uint8_t cc[16];
        int selc = 0;
        int sc = encode_at_scale(kind, sfmt, 16, xb, sbr, st, &cand[c], 1, 1, cc, &selc);
        double e = block_sse_sv(kind, sfmt, 16, xb, cc, sc, st, cand[c]);
        if (c == 0 || e < best) {
          best = e;
          sel = c;
          scode = sc;
          memcpy(cb, cc, 16);
        }
      }
    } else {
      scode = encode_at_scale(kind, sfmt, block, xb, sb_real, st, cand, ncand,
                              mode == RZO_MODE_RAZER, cb, &sel);
    }
    if (mode == RZO_MODE_FOUR_OVER_SIX) {
      /* [Four Over Six] Technical framework / key innovation: a block may
       * instead be scaled so that its maximum lands on 4 rather than 6 (block
       * scale 6/4 times larger); the block keeps whichever of the two plain
       * NVFP4 encodings has the smaller squared error in real units (ties keep
       * the usual max -> 6 scale). */
      uint8_t c4[128];
      int sel4 = 0;
      int scode4 = encode_at_scale(kind, sfmt, block, xb, sb_real * 1.5f, st, cand, ncand, 0, c4, &sel4);
      if (block_sse(kind, sfmt, block, xb, c4, scode4, st) <
          block_sse(kind, sfmt, block, xb, cb, scode, st)) {
        memcpy(cb, c4, (size_t)block);
        scode = scode4;
      }
    }
    if (scode == 0) continue; /* zero block: all +0, scale 0 */
    for (int j = 0; j < block / 2; j++)
      codes[(int64_t)block / 2 * b + j] = (uint8_t)(cb[2 * j] | (cb[2 * j + 1] << 4));
    /* Metadata in the freed scale bits ([notes] Key design 1 and the complete
     * example): the top bit = sign of the chosen special value; for weights
     * the next bit selects the pair (bits 7/6 of a byte scale, 15/14 of an
     * FP16 scale). */
    if (sfmt == RZO_SCALE_F16) {
      ((uint16_t*)scales)[b] = (uint16_t)(((sel & 1) << 15) | ((sel >> 1) << 14) | scode);
    } else {
      int meta = kind == RZO_WEIGHT ? (((sel & 1) << 7) | ((sel >> 1) << 6)) : (sel << 7);
      ((uint8_t*)scales)[b] = (uint8_t)(meta | scode);
    }
  }
  return 0;
}

double rzo_block_scale(int kind, int sbyte) {
  return kind == RZO_WEIGHT ? e3m3_value(sbyte & 63) : e4m3_value(sbyte & 127);
}

double rzo_decode_value(int kind, int code, int sbyte, const int8_t* off_half) {
  /* [notes] Key design 3 and the complete example: on the remapped code the
   * decoder reads the metadata, picks the offset register, forms 6 + offset
   * and attaches the sign; every other code is plain FP4. */
  if ((code & 15) == 8) {
    int neg = (sbyte >> 7) & 1;
    int pair = kind == RZO_WEIGHT ? (sbyte >> 6) & 1 : 0;
    return rzo_special_value(neg, off_half[pair]);
  }
  return rzo_fp4_value(code & 15);
}

static int code_at(const uint8_t* codes, int64_t idx) {
  uint8_t byte = codes[idx >> 1];
  return (idx & 1) ? (byte >> 4) : (byte & 15);
}

/* Value and block scale of element i of a tensor in either scale format. */
static void element_fmt(int kind, int sfmt, int block, const uint8_t* codes, const void* scales,
                        const int8_t* off_half, int64_t i, double* val, double* sb) {
  int code = code_at(codes, i);
  if (sfmt == RZO_SCALE_F16) {
    int sw = ((const uint16_t*)scales)[i / block];
    if ((code & 15) == 8) {
      int neg = (sw >> 15) & 1, pair = (sw >> 14) & 1;
      *val = rzo_special_value(neg, off_half[pair]);
    } else {
      *val = rzo_fp4_value(code & 15);
    }
    *sb = f16s_value(sw & 0x3FFF);
  } else {
    int sbyte = ((const uint8_t*)scales)[i / block];
    *val = rzo_decode_value(kind, code, sbyte, off_half);
    *sb = rzo_block_scale(kind, sbyte);
  }
}

void rzo_dequant_fmt_f64(int kind, int block, int sfmt, const uint8_t* codes, const void* scales,
                         float tensor_scale, const int8_t* off_half, int64_t rows, int64_t cols,
                         double* out) {
  int64_t n = rows * cols;
  for (int64_t i = 0; i < n; i++) {
    double v, sb;
    element_fmt(kind, sfmt, block, codes, scales, off_half, i, &v, &sb);
    out[i] = v * sb * (double)tensor_scale;
  }
}

void rzo_dequant_fmt_f32(int kind, int block, int sfmt, const uint8_t* codes, const void* scales,
                         float tensor_scale, const int8_t* off_half, int64_t rows, int64_t cols,
                         float* out) {
  int64_t n = rows * cols;
  for (int64_t i = 0; i < n; i++) {
    double v, sb;
    element_fmt(kind, sfmt, block, codes, scales, off_half, i, &v, &sb);
    /* value * block scale has at most 5 + 11 significant bits: exact in fp32 */
    float vs = (float)(v * sb);
    out[i] = vs * tensor_scale;
  }
}

void rzo_dequant_f64(int kind, const uint8_t* codes, const uint8_t* scales, float tensor_scale,
                     const int8_t* off_half, int64_t rows, int64_t cols, double* out) {
  rzo_dequant_fmt_f64(kind, 16, RZO_SCALE_BYTE, codes, scales, tensor_scale, off_half, rows, cols, out);
}

void rzo_dequant_f32(int kind, const uint8_t* codes, const uint8_t* scales, float tensor_scale,
                     const int8_t* off_half, int64_t rows, int64_t cols, float* out) {
  rzo_dequant_fmt_f32(kind, 16, RZO_SCALE_BYTE, codes, scales, tensor_scale, off_half, rows, cols, out);
}

void rzo_gemm(const float* x, int64_t m, int64_t k, int kind, const uint8_t* codes,
              const uint8_t* scales, float tensor_scale, const int8_t* off_half, int64_t n,
              const int64_t* cols_idx, int64_t ncols, double* y, double* norm) {
  double* w = (double*)malloc((size_t)(k > 0 ? k : 1) * sizeof(double));
  if (!w) return;
  for (int64_t jj = 0; jj < ncols; jj++) {
    int64_t j = cols_idx ? cols_idx[jj] : jj;
    if (j < 0 || j >= n) continue;
    /* decode weight row j exactly */
    for (int64_t kk = 0; kk < k; kk++) {
      int64_t idx = j * k + kk;
      int sbyte = scales[idx / 16];
      w[kk] = rzo_decode_value(kind, code_at(codes, idx), sbyte, off_half) *
              rzo_block_scale(kind, sbyte) * (double)tensor_scale;
    }
    for (int64_t i = 0; i < m; i++) {
      double acc = 0.0, nrm = 0.0;
      const float* xr = x + i * k;
      for (int64_t kk = 0; kk < k; kk++) {
        acc += (double)xr[kk] * w[kk];
        nrm += fabs((double)xr[kk]) * fabs(w[kk]);
      }
      y[i * ncols + jj] = acc;
      norm[i * ncols + jj] = nrm;
    }
  }
  free(w);
}
