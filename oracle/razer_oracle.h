/*
 * razer_oracle.h -- CPU oracle for RaZeR-NVFP4 (test infrastructure only).
 *
 * A plain, slow, single-threaded C statement of what the RaZeR-NVFP4 layer
 * computes: the two-level block-scaled FP4 encoder with redundant-zero
 * remapping, its decoder, and the W4A16 product.  It exists so that tests,
 * the smoke check and the bench's CPU-baseline leg have something obviously
 * correct to compare the GPU library against.  Nothing in the product path
 * may load it, and it shares no code, header, table or constant with the GPU
 * library (the two are written independently from the pages).
 *
 * Sources (page title, then the part of it used):
 *   [notes]   "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant
 *             Zero Remapping" (papernotes.org notes)
 *   [summary] "Technical Summary: RaZeR - Pushing the Limits of NVFP4
 *             Quantization with Redundant Zero Remapping" (gist.science)
 *   [Four Over Six] "Four Over Six: More Accurate NVFP4 Quantization with
 *             Adaptive Block Scaling" (the baseline encoder only)
 *
 * Pins (tests/test_oracle_pins.py): FP4 set, special-value rule, E4M3/E3M3
 * tables and rounding (torch float8_e4m3fn), FP4 rounding (closed form with
 * numpy rint), block argmin (exact rational brute force), error never above
 * plain NVFP4, product (numpy matmul).  Parity unpinned: the fp32 operation
 * order of the scale steps is a convention the pages do not fix; it is pinned
 * only up to fp32 rounding (scale codes equal the exact-rational nearest code
 * except within 2^-20 of a midpoint) and otherwise by GPU/CPU agreement.
 *
 * All pointers are host pointers.  Tensors are row-major [rows, cols]; blocks
 * are 16 consecutive elements of a row (cols must be a multiple of 16).
 * Packed layout: codes[r*cols/2 + i] = code(r,2i) | code(r,2i+1) << 4;
 * scales[r*cols/16 + b] = metadata bits | scale code.
 */
#ifndef RAZER_ORACLE_H
#define RAZER_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { RZO_WEIGHT = 0, RZO_ACT = 1 };

/* Encoder modes: plain NVFP4 (same scale format, no special value), RaZeR
 * (special-value remap), the Four Over Six baseline (plain FP4; each block
 * takes the max -> 6 or the max -> 4 block scale, whichever has the smaller
 * squared error in real units, ties to max -> 6), and RaZeR with rescaled
 * large special values: every candidate v is tried on its own, a candidate
 * with |v| > 6 at the block scale that maps the block maximum to |v| instead
 * of 6 (sb_real * 6 / |v| in fp32), the others at the usual scale; the block
 * keeps the candidate whose encoding has the smallest squared error in real
 * units (fp64, element order), ties to the lowest index.  This mode takes
 * 16-element blocks with byte scales only. */
enum { RZO_MODE_PLAIN = 0, RZO_MODE_RAZER = 1, RZO_MODE_FOUR_OVER_SIX = 2, RZO_MODE_RAZER_RESCALE = 3 };

/* Block-scale storage: one byte per block (E3M3 weights / E4M3 activations,
 * metadata in bits 7-6), or the group-scale variant for weights: a 16-bit FP16
 * scale per block whose sign bit and top exponent bit hold the metadata (bits
 * 15-14) and whose other 14 bits are the scale. */
enum { RZO_SCALE_BYTE = 0, RZO_SCALE_F16 = 1 };

/* FP4-E2M1 value of a 4-bit code (bit 3 = sign); code 8 is -0.0. */
double rzo_fp4_value(int code);
/* Index 0..7 of the FP4 magnitude nearest to a >= 0; ties go to the even index. */
int rzo_fp4_round_mag(double a);
/* Value of a block-scale code: E3M3 (kind = weight, code 0..63) or E4M3 (act, 0..126). */
double rzo_scale_value(int kind, int code);
/* Nearest block-scale code to v >= 0; ties go to the even code; saturates at the maximum. */
int rzo_scale_round(int kind, float v);
/* Largest block-scale value: 30 (E3M3) or 448 (E4M3). */
double rzo_scale_max(int kind);
/* The same three for either scale format (RZO_SCALE_*): the FP16 variant
 * holds 14-bit codes (exponent field 0..15), maximum 2 - 2^-10. */
double rzo_scale_value_fmt(int kind, int sfmt, int code);
int rzo_scale_round_fmt(int kind, int sfmt, float v);
double rzo_scale_max_fmt(int kind, int sfmt);
/* Special value selected by the metadata: (neg ? -1 : 1) * (6 + off_half/2). */
double rzo_special_value(int neg, int off_half);

/* Block remap on already-scaled values y[0..n): rounds each value to the FP4
 * grid, then (if remap) tries every candidate in cand[0..ncand) and keeps the
 * one with the lowest block squared error, ties to the lowest index.  Writes
 * one 4-bit code per element and the selected candidate index. */
void rzo_encode_block_scaled(const float* y, int n, const double* cand, int ncand,
                             int remap, uint8_t* codes, int* sel);

/* Full-tensor encode.  x: fp32 [rows, cols] (fp16/bf16 inputs are widened
 * exactly by the caller).  off_half: weight -> 2 entries, act -> 1 entry, each
 * in [-7, 7] (special value magnitude 6 + off/2).  mode: RZO_MODE_*; the plain
 * and Four Over Six modes never write the special-value code.  Returns 0, or
 * -1 on bad args. */
int rzo_quantize(int kind, const float* x, int64_t rows, int64_t cols,
                 const int8_t* off_half, int mode, uint8_t* codes, uint8_t* scales,
                 float* tensor_scale);

/* Block-size and scale-format variants ([notes] Key findings, block sizes 32,
 * 64 and 128; Key design 3, FP16 group scales): block in {16, 32, 64, 128}
 * elements along a row (cols % block == 0), sfmt RZO_SCALE_BYTE or (weights
 * only) RZO_SCALE_F16.  scales holds rows*cols/block entries of 1 or 2 bytes.
 * The tensor scale is amax / (6 * S_MAX) with S_MAX the format's largest scale.
 * In the Four Over Six mode a block's squared error is summed in fp64 in
 * element order.  rzo_quantize is this with block 16 and byte scales. */
int rzo_quantize_fmt(int kind, const float* x, int64_t rows, int64_t cols,
                     const int8_t* off_half, int mode, int block, int sfmt, uint8_t* codes,
                     void* scales, float* tensor_scale);
void rzo_dequant_fmt_f64(int kind, int block, int sfmt, const uint8_t* codes, const void* scales,
                         float tensor_scale, const int8_t* off_half, int64_t rows, int64_t cols,
                         double* out);
void rzo_dequant_fmt_f32(int kind, int block, int sfmt, const uint8_t* codes, const void* scales,
                         float tensor_scale, const int8_t* off_half, int64_t rows, int64_t cols,
                         float* out);

/* Decoded value (no scaling) of element code `code` in a block with scale byte `sbyte`. */
double rzo_decode_value(int kind, int code, int sbyte, const int8_t* off_half);
/* Block scale value held in scale byte `sbyte` (metadata bits stripped). */
double rzo_block_scale(int kind, int sbyte);

/* Dequantize: out64 exact (val*sb*st in fp64); out32 = fl32(fl32(val*sb)*st). */
void rzo_dequant_f64(int kind, const uint8_t* codes, const uint8_t* scales, float tensor_scale,
                     const int8_t* off_half, int64_t rows, int64_t cols, double* out);
void rzo_dequant_f32(int kind, const uint8_t* codes, const uint8_t* scales, float tensor_scale,
                     const int8_t* off_half, int64_t rows, int64_t cols, float* out);

/* W4A16 product y[i, j] = sum_k x[i, k] * w[col_j, k] accumulated in fp64,
 * and norm[i, j] = sum_k |x[i, k]| * |w[col_j, k]|, for the weight rows listed
 * in cols_idx (NULL = all n rows, in order).  x: fp32 [m, k]; weight packed
 * [n, k].  y and norm: [m, ncols]. */
void rzo_gemm(const float* x, int64_t m, int64_t k, int kind, const uint8_t* codes,
              const uint8_t* scales, float tensor_scale, const int8_t* off_half, int64_t n,
              const int64_t* cols_idx, int64_t ncols, double* y, double* norm);

#ifdef __cplusplus
}
#endif
#endif
