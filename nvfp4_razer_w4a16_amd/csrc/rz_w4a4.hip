// rz_w4a4.hip -- W4A4 product y[M, N] = dequant(x)[M, K] * dequant(w)^T of two
// RaZeR-packed tensors on gfx950.
//
// "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
// Remapping" (papernotes.org notes), Overall framework and Key designs 1-2:
// activations carry the online 2-candidate encoding (E4M3 block scale), weights
// the offline 4-candidate one; the product runs over the decoded values.  On
// matrix units without an FP4 path the activations are decoded first:
//   1. x's codes become value * sb in fp16, exactly: FP4 values and the special
//      values +/-(6 + off/2) have at most 5 significant bits, a block scale 4,
//      so at most 9 of fp16's 11, and |value * sb| lies in [2^-10, 9.5 * 448];
//   2. the W4A16 product runs on that fp16 matrix into an fp32 buffer
//      (y32 = st_w * sum(...));
//   3. y = y32 * st_x, rounded once to the output type.
// For prefill shapes passes 2 and 3 are one: the product's epilogue multiplies
// by st_w, then by st_x, and rounds once (the same operations in the same
// order).  Every pass is one of this library's kernels; the workspace holds the
// fp16 activations, the fp32 product and the product's own workspace (prefill
// shapes: the fp16 activations and the product's workspace).
#include "rz_device.h"
#include "rz_launch.h"

namespace rz {

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

template <typename OT> __device__ __forceinline__ OT cvt_out(float v);
template <> __device__ __forceinline__ float cvt_out<float>(float v) { return v; }
template <> __device__ __forceinline__ _Float16 cvt_out<_Float16>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ __bf16 cvt_out<__bf16>(float v) { return (__bf16)v; }

template <typename OT>
__global__ __launch_bounds__(256) void scale_out_kernel(const float* __restrict__ y32, int64_t n,
                                                        const float* __restrict__ st_x, OT* __restrict__ y) {
  const float s = *st_x;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    y[i] = cvt_out<OT>(y32[i] * s);
}

size_t product_ws(int64_t m, int64_t n, int64_t k) { return m == 1 ? gemv_ws_bytes(n, k) : gemm_ws_bytes(m, n, k); }

}  // namespace

size_t gemm_w4a4_ws_bytes(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0) return 0;
  // prefill shapes write y from the product's epilogue: no fp32 product buffer
  if (gemm_prefill_fits(m, k, kF16)) return up((size_t)m * (size_t)k * 2) + up(prefill_ws_bytes(m, n, k));
  return up((size_t)m * (size_t)k * 2) + up((size_t)m * (size_t)n * 4) + up(product_ws(m, n, k));
}

hipError_t launch_gemm_w4a4(const PackedView& x, const PackedView& w, void* y, int y_dtype, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  const int64_t m = x.rows, k = x.cols, n = w.rows;
  if (m == 0 || n == 0) return hipSuccess;
  uint8_t* base = (uint8_t*)ws;
  void* xb = base;  // fp16 [m, k]
  const size_t xb_bytes = up((size_t)m * k * 2);
  hipError_t e = launch_dequant_unscaled(x, xb, kF16, stream);
  if (e != hipSuccess) return e;
  // prefill shapes: the product's epilogue applies st_x after st_w and writes
  // y directly -- the same two fp32 multiplies and one rounding as passes 2-3;
  // the rest of the workspace serves the product's tail split
  if (gemm_prefill_fits(m, k, kF16))
    return launch_gemm_prefill_scaled(xb, kF16, m, w, y, y_dtype, x.tensor_scale, base + xb_bytes,
                                      ws_bytes - xb_bytes, stream);
  float* y32 = (float*)(base + xb_bytes);  // fp32 [m, n]
  void* pws = base + xb_bytes + up((size_t)m * n * 4);
  const size_t pws_bytes = ws_bytes - (xb_bytes + up((size_t)m * n * 4));
  e = m == 1 ? launch_gemv(xb, kF16, w, y32, kF32, pws, pws_bytes, stream)
             : launch_gemm(xb, kF16, m, w, y32, kF32, pws, pws_bytes, stream);
  if (e != hipSuccess) return e;
  const int64_t total = m * n;
  int64_t g = (total + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (g > cap) g = cap;
  if (y_dtype == kF32)
    hipLaunchKernelGGL(scale_out_kernel<float>, dim3((unsigned)g), dim3(256), 0, stream, y32, total,
                       x.tensor_scale, (float*)y);
  else if (y_dtype == kF16)
    hipLaunchKernelGGL(scale_out_kernel<_Float16>, dim3((unsigned)g), dim3(256), 0, stream, y32, total,
                       x.tensor_scale, (_Float16*)y);
  else
    hipLaunchKernelGGL(scale_out_kernel<__bf16>, dim3((unsigned)g), dim3(256), 0, stream, y32, total,
                       x.tensor_scale, (__bf16*)y);
  return hipGetLastError();
}

}  // namespace rz
