/*
 * librazer.h -- C ABI of librazer, the RaZeR-NVFP4 W4A16 layer for AMD MI355X
 * (CDNA4, gfx950).
 *
 * Sources cited below (page title, then section):
 *   [notes]   "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant
 *             Zero Remapping" (papernotes.org notes)
 *   [summary] "Technical Summary: RaZeR - Pushing the Limits of NVFP4
 *             Quantization with Redundant Zero Remapping" (gist.science)
 *
 * THE FORMAT ([notes] Background, Overall framework, Key design 1-3;
 * [summary] §2.1-2.2).  A tensor X[rows, cols] (row-major, cols % 16 == 0) is
 * cut into 16-element blocks along each row.  It carries one FP32 tensor
 * scale st and, per block, one scale byte and 16 four-bit element codes:
 *
 *   st       = amax(|X|) / (6 * S_MAX)                       (fp32)
 *   sb_code  = round_nearest_even(S_MAX * amax_block / amax(|X|))
 *              onto E3M3 (weights: 3 exp bits, bias 3, max 30) or
 *              E4M3 (activations: OCP E4M3FN, max 448)
 *   y_j      = x_j * (1 / (sb * st))                         (fp32)
 *   code_j   = FP4-E2M1 of y_j: sign bit 3, magnitude index 0..7 of
 *              {0, 0.5, 1, 1.5, 2, 3, 4, 6}, nearest-even, saturating at 6;
 *              zero is always written as +0 (0b0000)
 *   The redundant -0 code 0b1000 is remapped to a per-block special value
 *   SV = sign * (6 + off/2).  Each block keeps the candidate with the lowest
 *   block squared error ([notes] Key design 2, block MSE equation), ties to
 *   the lowest candidate index; an element takes SV only if SV is strictly
 *   nearer than its FP4 rounding.
 *     weights:     4 candidates +M0, -M0, +M1, -M1 (two +/- pairs),
 *                  scale byte = sign << 7 | pair << 6 | E3M3 code (6 bits)
 *     activations: 2 candidates +M0, -M0,
 *                  scale byte = sign << 7 | E4M3 code (7 bits)
 *   with M_i = 6 + sv_off_half[i] / 2 ([notes] Key design 3: 4-bit offset
 *   registers holding [-3.5, 3.5] in steps of 0.5).
 *
 * MEMORY LAYOUT of a packed tensor (all device memory, caller-owned):
 *   codes[r * cols/2 + i]   = code(r, 2i) | code(r, 2i+1) << 4   (u8)
 *   scales[r * cols/16 + b] = scale byte of block b of row r     (u8)
 *   tensor_scale[0]         = st                                 (fp32)
 * A weight W[N, K] is stored like a PyTorch Linear weight (row n holds the K
 * inputs of output n); products compute y[M, N] = x[M, K] * W^T.
 *
 * CONVENTIONS for every call:
 *   - Pointers marked "device" point to GPU memory on the current HIP device.
 *     The caller allocates and frees every buffer, including workspaces; the
 *     library never allocates, frees or synchronises, and keeps no mutable
 *     global state, except the 4 KiB per-device scratch array of
 *     razer_quantize_act_noalloc.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued on it, asynchronously, in stream order.
 *   - Host-side argument checks are synchronous: on RAZER_E_INVALID or
 *     RAZER_E_UNSUPPORTED nothing is enqueued and nothing is written.
 *     RAZER_E_HIP reports a failed kernel launch.
 *   - Data errors are reported through data, not status: a non-finite input
 *     element makes the encoder write tensor_scale = NaN and all codes and
 *     scale bytes 0; a product whose weight has a NaN tensor scale outputs NaN.
 *   - Device pointers must be 16-byte aligned (x, w, y, codes) and 4-byte
 *     aligned (scales, tensor_scale, workspace).
 *   - Calls on different streams may run concurrently if they write disjoint
 *     buffers (including workspaces).
 */
#ifndef LIBRAZER_H
#define LIBRAZER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The two enums below carry range markers so that every 32-bit value a C
 * caller may pass is a valid value of the type (the library rejects the ones
 * that are not a listed constant). */
typedef enum razer_status {
  RAZER_OK = 0,
  RAZER_E_INVALID = 1,     /* bad argument: null pointer, shape, alignment, offsets, workspace */
  RAZER_E_UNSUPPORTED = 2, /* valid but not implemented (dtype/kind/shape combination) */
  RAZER_E_HIP = 3,         /* the HIP runtime refused a launch */
  RAZER_STATUS_RANGE_MIN_ = -0x7FFFFFFF - 1,
  RAZER_STATUS_RANGE_MAX_ = 0x7FFFFFFF
} razer_status;

typedef enum razer_dtype {
  RAZER_F32 = 0,
  RAZER_F16 = 1,
  RAZER_BF16 = 2,
  RAZER_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
  RAZER_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} razer_dtype;

/* Which scale format and candidate set a packed tensor uses ([notes] Key
 * design 1: weights free 2 scale bits, activations 1). */
typedef enum razer_kind { RAZER_WEIGHT = 0, RAZER_ACT = 1 } razer_kind;

/* flags of razer_packed */
enum {
  /* Encode as plain NVFP4 (no special value; sel = 0 everywhere) with the same
   * scale format: the comparator of the pages' main table, used to measure
   * what the special-value search costs ([notes] Key design 2 states the
   * activation search adds under 2% to quantizer time). */
  RAZER_FLAG_NO_REMAP = 1u,
  /* Encode with the Four Over Six baseline (page "Four Over Six: More Accurate
   * NVFP4 Quantization with Adaptive Block Scaling", technical framework and
   * key innovation): plain FP4 (no special value), and each block takes the
   * block scale whose code is nearest to S_MAX * amax_block / amax_tensor
   * (max -> 6) or to 1.5 times that (max -> 4, saturating at the format
   * maximum), whichever gives the smaller squared error against the input in
   * real units (summed in fp64 in element order; a tie keeps max -> 6).  The
   * tensor scale and the packed layout are unchanged, so every decoding call
   * reads such a tensor as plain NVFP4.  Takes precedence over NO_REMAP.
   * The quantize calls reject any other flag bit than these three with
   * RAZER_E_INVALID. */
  RAZER_FLAG_FOUR_OVER_SIX = 2u,
  /* Read by the product calls only (the encoders reject it): launch the
   * product with the untrimmed plan -- the K range split over the most waves
   * or workgroups the kernel allows and the fewest rows per wave, so every CU
   * gets work however small the matrix -- instead of the launch plan sized
   * per shape.  For measuring what the launch sizing gains: the counterpart
   * of the pages' adaptive trimming of SM launches for small matrices ([notes]
   * Key design 3).  Outputs agree within the product tolerance (the
   * summation order changes).  razer_gemm then needs
   * razer_workspace_bytes(RAZER_OP_GEMM_UNTRIMMED, ...). */
  RAZER_FLAG_UNTRIMMED_PLAN = 4u,
  /* Encode with rescaled large special values (a reading of [notes] Training
   * strategy, whose best weight pairs include +/-7, +/-8 and +/-9, values a
   * block scaled so that its maximum maps to 6 almost never reaches): every
   * candidate special value v is tried on its own -- one with |v| > 6 at the
   * block scale whose code is nearest to S_MAX * amax_block / amax_tensor *
   * 6 / |v| (fp32: (sb_real * 6) / |v|), so the block maximum maps to |v|, the
   * others at the usual scale -- and the block keeps the encoding with the
   * smallest squared error against the input in real units (fp64, element
   * order; ties to the lowest candidate index).  Decoding is unchanged (the
   * scale byte holds the chosen scale and the metadata the chosen value).
   * 16-element blocks with byte scales only (other layouts:
   * RAZER_E_UNSUPPORTED); NO_REMAP and FOUR_OVER_SIX take precedence. */
  RAZER_FLAG_RESCALE_LARGE_SV = 8u
};

/* Block-scale storage of a packed tensor (razer_packed.scale_fmt). */
enum {
  /* One byte per block: E3M3 (weights) / E4M3 (activations) scale code with
   * the metadata in bits 7-6 ([notes] Key design 1).  The default. */
  RAZER_SCALE_BYTE = 0,
  /* Weights only: one 16-bit FP16 scale per block whose sign bit and top
   * exponent bit hold the metadata (bit 15 = sign of the special value, bit
   * 14 = pair) and whose other 14 bits are the scale, an FP16 number with
   * exponent field 0..15, at most 2 - 2^-10 ([notes] Key design 3: the
   * layout of the pages' Blackwell kernels, there with 128-element blocks).
   * The tensor scale is amax / (6 * (2 - 2^-10)). */
  RAZER_SCALE_F16 = 1
};

typedef struct razer_packed {
  int32_t kind;          /* razer_kind */
  uint32_t flags;        /* RAZER_FLAG_* (encoder flags; RAZER_FLAG_UNTRIMMED_PLAN for products) */
  int64_t rows;          /* >= 0 */
  int64_t cols;          /* >= 0, multiple of the block size */
  int8_t sv_off_half[2]; /* special-value offsets in units of 0.5, each in [-7, 7];
                            weights use both, activations use [0] only */
  uint8_t block_log2;    /* elements per block = 2^block_log2, 4..7 (16..128, [notes]
                            Key findings: block sizes 32, 64, 128); 0 reads as 4 */
  uint8_t scale_fmt;     /* RAZER_SCALE_BYTE or RAZER_SCALE_F16 */
  int8_t reserved[4];
  uint8_t* codes;        /* device, rows*cols/2 bytes */
  uint8_t* scales;       /* device, rows*cols/block entries of 1 (byte) or 2 (F16) bytes */
  float* tensor_scale;   /* device, 1 float */
} razer_packed;
/* The encoders and razer_dequant take every layout.  The product calls take
 * 16-element blocks with byte scales; razer_gemv, razer_gemv_group (all
 * members in one layout) and razer_gemm (any m) also take the pages' kernel
 * layout, 128-element blocks (block_log2 7) with RAZER_SCALE_F16.  Other
 * layouts, and any layout but the default for razer_gemm_w4a4, return
 * RAZER_E_UNSUPPORTED. */

/* Operation ids for razer_workspace_bytes. */
enum {
  RAZER_OP_QUANTIZE_WEIGHT = 0,
  RAZER_OP_QUANTIZE_ACT = 1,
  RAZER_OP_GEMV = 2,
  RAZER_OP_GEMM = 3,
  RAZER_OP_OFFSET_SEARCH = 4, /* n = rows, k = cols of the weight */
  RAZER_OP_GEMM_W4A4 = 5,     /* m = rows of x, n = rows of w, k = cols */
  RAZER_OP_GEMM_UNTRIMMED = 6 /* razer_gemm of a weight with RAZER_FLAG_UNTRIMMED_PLAN */
};

/* Offline weight encoder: 4-candidate block-MSE search ([notes] Key design 2:
 * weights are searched offline over two +/- pairs; [summary] §2.2).
 * w: device [out->rows, out->cols] in w_dt (F32, F16 or BF16).  out: describes
 * the destination; kind must be RAZER_WEIGHT; codes/scales/tensor_scale are
 * written.  ws: device workspace of at least
 * razer_workspace_bytes(RAZER_OP_QUANTIZE_WEIGHT, rows, 0, cols) bytes. */
razer_status razer_quantize_weight(const void* w, razer_dtype w_dt, const razer_packed* out,
                                   void* ws, size_t ws_bytes, void* stream);

/* Online activation encoder: 2 candidates +/-M0 with the E4M3 block scale
 * ([notes] Key design 1 and 2; [summary] §2.2).  x: device [rows, cols] in
 * F16 or BF16 (F32 also accepted).  out->kind must be RAZER_ACT. */
razer_status razer_quantize_act(const void* x, razer_dtype x_dt, const razer_packed* out,
                                void* ws, size_t ws_bytes, void* stream);

/* razer_quantize_act without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments (minus ws / ws_bytes), checks and
 * output bytes as razer_quantize_act.  The amax partials live in a 4 KiB
 * static device array that the library holds on each device it runs on until
 * the process ends; the first call on a device resolves that array's address
 * (hipGetSymbolAddress), so make it outside stream capture.  Every call on one
 * device shares the array: calls that overlap on one device (different
 * streams, concurrent graph launches) race and must be ordered by the caller.
 * The array is large enough for every input size (the partials never exceed
 * it); RAZER_E_UNSUPPORTED would report a build where they did.  Allocates
 * nothing, frees nothing, synchronises nothing. */
razer_status razer_quantize_act_noalloc(const void* x, razer_dtype x_dt, const razer_packed* out,
                                        void* stream);

/* Decode a packed tensor ([notes] Key design 3 decoder): out[r, c] =
 * value(code) * sb * st, with value(0b1000) = (bit7 ? -1 : 1) * (6 + off/2).
 * F32 output is fl32(fl32(value * sb) * st); F16/BF16 output is that fp32
 * value rounded to nearest even.  out: device [rows, cols] in out_dt. */
razer_status razer_dequant(const razer_packed* t, void* out, razer_dtype out_dt, void* stream);

/* Batch-1 W4A16 product y[1, N] = x[1, K] * W^T with W decoded in registers
 * ([notes] Key design 3: weight-only GEMV kernels; [summary] §2.3).
 * x: device [K] in F16 or BF16.  w: packed tensor [N, K] of either kind
 * (weights, or an activation encoding used as the right operand).  y: device [N] in
 * F32, F16 or BF16.  Accumulation is fp32.  ws: at least
 * razer_workspace_bytes(RAZER_OP_GEMV, 1, N, K) bytes (may be 0 -> ws NULL). */
razer_status razer_gemv(const void* x, razer_dtype x_dt, const razer_packed* w, void* y,
                        razer_dtype y_dt, void* ws, size_t ws_bytes, void* stream);

/* Largest count accepted by razer_gemv_group. */
#define RAZER_GEMV_GROUP_MAX 4

/* Several batch-1 products that share one input vector, y_g[1, N_g] = x[1, K] *
 * W_g^T for g < count, in one launch where the GEMV kernel serves them (the
 * product of razer_gemv for each weight, [notes] Key design 3; sharing the
 * launch is the counterpart of the pages' launch sizing for small matrices:
 * two weights of one input, such as an MLP's gate and up projections, cost
 * one launch and one ramp instead of two).  x: device [K] in F16 or BF16.
 * w: host array of count packed-tensor descriptors (either kind, each with its
 * own tensor scale and offsets) with equal cols K.  y: host array of count
 * device outputs [N_g] in y_dt (16-byte aligned; may be NULL where N_g == 0).
 * 1 <= count <= RAZER_GEMV_GROUP_MAX.  Each y_g is bitwise what razer_gemv
 * writes for W_g.  No workspace.  Errors: RAZER_E_INVALID for a bad count,
 * unequal K or any argument razer_gemv would reject; RAZER_E_UNSUPPORTED as
 * for razer_gemv. */
razer_status razer_gemv_group(const void* x, razer_dtype x_dt, const razer_packed* const* w,
                              void* const* y, int count, razer_dtype y_dt, void* stream);

/* Batched W4A16 product y[M, N] = x[M, K] * W^T ([notes] Key design 3;
 * [summary] §2.3: weight-only GEMM kernels for small and large batches).
 * x: device [m, K] row-major in F16 or BF16.  w: packed tensor [N, K] of either
 * kind, default layout or 128-element blocks with FP16 scales.  y: device
 * [m, N] in F32, F16 or BF16.  m >= 1; m == 1 runs the GEMV path.  ws: at least
 * razer_workspace_bytes(RAZER_OP_GEMM, m, N, K) bytes (enough for either
 * layout).  For m >= 256 (the 256x256-tile kernel) the workspace is optional:
 * NULL, smaller or not 16-byte aligned, the product runs without it; with it,
 * when the tile count leaves a last round of tiles on at most half of the
 * compute units, those tiles are computed as two K halves (fp32 partial tiles
 * in ws, then added in one more launch). */
razer_status razer_gemm(const void* x, razer_dtype x_dt, int64_t m, const razer_packed* w, void* y,
                        razer_dtype y_dt, void* ws, size_t ws_bytes, void* stream);

/* W4A4 product y[M, N] = dequant(x)[M, K] * dequant(w)^T of two packed
 * tensors ([notes] Overall framework, Key designs 1-2: activations encoded
 * online with 2 candidates, weights offline with 4).  On matrix units without
 * an FP4 path it runs in two passes: x's codes are decoded to value * sb in
 * fp16 (exact), the W4A16 product runs on them in fp32, and the result is
 * multiplied by x's tensor scale and rounded once to y_dt.  x: packed [M, K]
 * (normally RAZER_ACT, either kind accepted); w: packed [N, K] of either kind;
 * y: device [M, N] in F32, F16 or BF16.  K == 0 is RAZER_E_UNSUPPORTED.
 * ws: at least razer_workspace_bytes(RAZER_OP_GEMM_W4A4, M, N, K) bytes,
 * 256-byte aligned.  The accuracy bound is the W4A16 product's plus one fp32
 * rounding. */
razer_status razer_gemm_w4a4(const razer_packed* x, const razer_packed* w, void* y, razer_dtype y_dt,
                             void* ws, size_t ws_bytes, void* stream);

/* Second-pair offset search for the offline weight encoder ([notes] Loss
 * function / training strategy: the extra weight pair is picked offline by a
 * grid search).  For each offset o = -7..7 of the second pair, the weight is
 * encoded exactly as razer_quantize_weight would with offsets (off0_half, o),
 * and sse[o + 7] receives sum((w - value * sb * st)^2) over the tensor,
 * accumulated in fp64 (value * sb * st is exact in fp64).  The caller picks
 * the offset (e.g. the lowest sse, ties to the lowest offset) and passes it to
 * razer_quantize_weight.  w: device [rows, cols] in w_dt (F32, F16, BF16),
 * cols % 16 == 0.  sse: device, 15 doubles, 8-byte aligned.  A non-finite
 * weight gives NaN in all 15; an all-zero or empty weight gives 0.  ws: at
 * least razer_workspace_bytes(RAZER_OP_OFFSET_SEARCH, 0, rows, cols) bytes,
 * 8-byte aligned.  Summation order is fixed, so results repeat bit for bit. */
razer_status razer_weight_offset_sse(const void* w, razer_dtype w_dt, int64_t rows, int64_t cols,
                                     int off0_half, double* sse, void* ws, size_t ws_bytes,
                                     void* stream);

/* Workspace bytes an operation needs for the given sizes (m rows of x, n
 * weight rows / output features, k reduction length).  0 means none.  For
 * RAZER_OP_GEMM with m >= 256 the figure is what the prefill kernel's tail
 * split uses (it depends on the current device's compute-unit count); that
 * workspace is optional there. */
size_t razer_workspace_bytes(int op, int64_t m, int64_t n, int64_t k);

/* Static, human-readable name of a status code. */
const char* razer_status_string(razer_status s);

#ifdef __cplusplus
}
#endif
#endif /* LIBRAZER_H */
