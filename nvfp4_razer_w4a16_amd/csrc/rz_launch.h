// rz_launch.h -- internal launcher interface between the C ABI layer and the
// kernel translation units.  Host-only declarations; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rz {

// Encoder flags (the values of the public RAZER_FLAG_* constants).
constexpr uint32_t kFlagNoRemap = 1u;       // plain NVFP4: no special value
constexpr uint32_t kFlagFourOverSix = 2u;   // plain FP4, per-block max -> 6 or max -> 4 scale
constexpr uint32_t kFlagUntrimmed = 4u;     // products: untrimmed launch plan (most splits)
constexpr uint32_t kFlagRescale = 8u;       // encoders: candidates with |SV| > 6 rescale the block (max -> |SV|)

struct PackedView {
  int kind;          // 0 weight (E3M3, 4 candidates), 1 activation (E4M3, 2 candidates)
  uint32_t flags;    // kFlag* bits
  int64_t rows, cols;
  int off_half[2];   // special-value offsets in units of 0.5
  int blog2 = 4;     // log2 of the elements per block (4..7)
  int sfmt = 0;      // 0: byte scales (E3M3 / E4M3); 1: FP16 group scales (weights)
  uint8_t* codes;
  uint8_t* scales;
  float* tensor_scale;
};

// Special-value candidate magnitudes M = 6 + off/2 and the open interval
// (lo, hi) of |y| values that move to M instead of their FP4 rounding.
struct Candidate {
  float mag;       // M
  float lo, hi;    // lo < |y| < hi moves to M; lo = hi = 0 when M is an FP4 value
  int mag_x2;      // 2 * M (integer)
};
Candidate make_candidate(int off_half);

// Quantizer: partial tensor-amax pass + block encode pass.
constexpr int kAmaxMaxPartials = 1024;
size_t quantize_ws_bytes();
hipError_t launch_quantize(const void* x, int dtype, const PackedView& out, void* ws,
                           hipStream_t stream);
// The same with the partials in a static per-device array (no workspace).
size_t noalloc_scratch_bytes();
hipError_t launch_quantize_noalloc(const void* x, int dtype, const PackedView& out, hipStream_t stream);

// Second-pair offset search: sse[o + 7] = total fp64 squared error of the
// weight tensor encoded with offsets (off0, o), o = -7..7.
size_t offset_search_ws_bytes(int64_t n);
hipError_t launch_offset_search(const void* x, int dtype, int64_t rows, int64_t cols, int off0,
                                double* sse, void* ws, hipStream_t stream);

hipError_t launch_dequant(const PackedView& t, void* out, int out_dtype, hipStream_t stream);
hipError_t launch_dequant_unscaled(const PackedView& t, void* out, int out_dtype, hipStream_t stream);

// W4A4 product of two packed tensors (two passes through the W4A16 product).
size_t gemm_w4a4_ws_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_w4a4(const PackedView& x, const PackedView& w, void* y, int y_dtype, void* ws,
                            size_t ws_bytes, hipStream_t stream);

size_t gemv_ws_bytes(int64_t n, int64_t k);
// Up to four weights with the same K and one input x in one launch
// (members that the small-batch kernel serves better are launched on their own).
hipError_t launch_gemv_group(const void* x, int x_dtype, const PackedView* w, void* const* y,
                             int count, int y_dtype, hipStream_t stream);
// The layout every product kernel reads: 16-element blocks, byte scales.
inline bool default_layout(const PackedView& v) { return v.blog2 == 4 && v.sfmt == 0; }

// The prefill (M >= 256, K % 64 == 0) product with a second scale factor
// applied after the weight's tensor scale in the epilogue.  ws (optional, at
// least prefill_ws_bytes) holds the partial tiles of the last round's K split.
bool gemm_prefill_fits(int64_t m, int64_t k, int x_dtype);
size_t prefill_ws_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_prefill_scaled(const void* x, int x_dtype, int64_t m, const PackedView& w, void* y,
                                      int y_dtype, const float* ts2, void* ws, size_t wsb, hipStream_t stream);
hipError_t launch_gemv(const void* x, int x_dtype, const PackedView& w, void* y, int y_dtype,
                       void* ws, size_t ws_bytes, hipStream_t stream);

// MFMA kernel for 1..4 activation rows (K a multiple of 256 / M rounded up to
// 1, 2, 4); returns hipErrorNotSupported for shapes it does not cover.
bool smallm_supported(int64_t m, int64_t n, int64_t k);
hipError_t launch_smallm(const void* x, int x_dtype, int64_t m, const PackedView& w, void* y,
                         int y_dtype, hipStream_t stream);

// Block-diagonal MFMA kernel for 2..8 activation rows (default layout,
// K % 256 == 0); no workspace.
bool bdiag_supported(int64_t m, int64_t n, int64_t k);
// The same kernel on the FP16-scale layout (2..32 rows, dense x tiles above 8).
bool fp16s_supported(int64_t m, int64_t n, int64_t k);
hipError_t launch_bdiag(const void* x, int x_dtype, int64_t m, const PackedView& w, void* y, int y_dtype,
                        hipStream_t stream);

size_t gemm_ws_bytes(int64_t m, int64_t n, int64_t k);                // either layout
size_t gemm_ws_need(int64_t m, int64_t n, int64_t k, bool f16s, bool untrimmed = false);  // one layout
hipError_t launch_gemm(const void* x, int x_dtype, int64_t m, const PackedView& w, void* y,
                       int y_dtype, void* ws, size_t ws_bytes, hipStream_t stream);

// Device properties used for launch sizing (cached per device).
int device_cu_count();

}  // namespace rz
