// rz_gemv.hip -- batch-1 W4A16 product y = x * W^T on gfx950, decoding the
// RaZeR weight format in registers.
//
// "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
// Remapping" (papernotes.org notes), Key design 3: weight-only GEMV kernels
// decode the packed weights inside the kernel, and the launch is trimmed so
// small matrices are not over-split; "Technical Summary: RaZeR ..."
// (gist.science), §2.3.  The pages' kernel (group-128 FP16 scales on another
// GPU) is prior art only; this one is written for CDNA4:
//   - one wavefront owns one weight row at a time; lane l walks 32-element
//     chunks l, l+64, ... so each 16-byte code load is fully coalesced;
//   - x is staged once per workgroup in LDS, together with a 256-entry table
//     of (sb, sb * SV / 2) indexed by the scale byte;
//   - codes become fp16/bf16 pairs with the gfx950 packed FP4 conversion and
//     are contracted with x by v_dot2 (fp32 accumulate).  The remapped -0 code
//     converts to -0 and contributes nothing there; a second pass turns the
//     remapped positions into FP4 +2.0 and dots them with x, and the block sum
//     is dot * sb + special_dot * (sb * SV / 2);
//   - the 64 lane partials of a row are summed with cross-lane shuffles and
//     scaled once by the tensor scale.
#include "rz_device.h"
#include "rz_launch.h"

namespace rz {

template <typename XT> struct Pair;
template <> struct Pair<_Float16> {
  typedef half2_t T;
  static __device__ __forceinline__ float dot(T a, T b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
  }
};
template <> struct Pair<__bf16> {
  typedef bf162_t T;
  static __device__ __forceinline__ float dot(T a, T b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
};

// FP4 pair (byte `sel` of w: low nibble -> element 0) to two 16-bit floats.
#define RZ_CVT_F16(w, s) __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((w), 1.0f, (s))
#define RZ_CVT_BF16(w, s) __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((w), 1.0f, (s))

template <typename OT> __device__ __forceinline__ OT gemv_out(float v);
template <> __device__ __forceinline__ float gemv_out<float>(float v) { return v; }
template <> __device__ __forceinline__ _Float16 gemv_out<_Float16>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ __bf16 gemv_out<__bf16>(float v) { return (__bf16)v; }

// Contract one 16-element block: codes w0 (elements 0..7), w1 (8..15) with the
// 8 x pairs at xp.  Returns the FP4 dot and the remapped-position dot (x2).
template <typename XT>
__device__ __forceinline__ void block_dot(uint32_t w0, uint32_t w1, const typename Pair<XT>::T* xp,
                                          float& d, float& s) {
  const uint32_t o0 = special_onehot_x2(w0), o1 = special_onehot_x2(w1);
  d = 0.0f;
  s = 0.0f;
  if constexpr (sizeof(XT) == 2 && __is_same(XT, _Float16)) {
    d = Pair<XT>::dot(RZ_CVT_F16(w0, 0), xp[0], d);
    d = Pair<XT>::dot(RZ_CVT_F16(w0, 1), xp[1], d);
    d = Pair<XT>::dot(RZ_CVT_F16(w0, 2), xp[2], d);
    d = Pair<XT>::dot(RZ_CVT_F16(w0, 3), xp[3], d);
    d = Pair<XT>::dot(RZ_CVT_F16(w1, 0), xp[4], d);
    d = Pair<XT>::dot(RZ_CVT_F16(w1, 1), xp[5], d);
    d = Pair<XT>::dot(RZ_CVT_F16(w1, 2), xp[6], d);
    d = Pair<XT>::dot(RZ_CVT_F16(w1, 3), xp[7], d);
    s = Pair<XT>::dot(RZ_CVT_F16(o0, 0), xp[0], s);
    s = Pair<XT>::dot(RZ_CVT_F16(o0, 1), xp[1], s);
    s = Pair<XT>::dot(RZ_CVT_F16(o0, 2), xp[2], s);
    s = Pair<XT>::dot(RZ_CVT_F16(o0, 3), xp[3], s);
    s = Pair<XT>::dot(RZ_CVT_F16(o1, 0), xp[4], s);
    s = Pair<XT>::dot(RZ_CVT_F16(o1, 1), xp[5], s);
    s = Pair<XT>::dot(RZ_CVT_F16(o1, 2), xp[6], s);
    s = Pair<XT>::dot(RZ_CVT_F16(o1, 3), xp[7], s);
  } else {
    d = Pair<XT>::dot(RZ_CVT_BF16(w0, 0), xp[0], d);
    d = Pair<XT>::dot(RZ_CVT_BF16(w0, 1), xp[1], d);
    d = Pair<XT>::dot(RZ_CVT_BF16(w0, 2), xp[2], d);
    d = Pair<XT>::dot(RZ_CVT_BF16(w0, 3), xp[3], d);
    d = Pair<XT>::dot(RZ_CVT_BF16(w1, 0), xp[4], d);
    d = Pair<XT>::dot(RZ_CVT_BF16(w1, 1), xp[5], d);
    d = Pair<XT>::dot(RZ_CVT_BF16(w1, 2), xp[6], d);
    d = Pair<XT>::dot(RZ_CVT_BF16(w1, 3), xp[7], d);
    s = Pair<XT>::dot(RZ_CVT_BF16(o0, 0), xp[0], s);
    s = Pair<XT>::dot(RZ_CVT_BF16(o0, 1), xp[1], s);
    s = Pair<XT>::dot(RZ_CVT_BF16(o0, 2), xp[2], s);
    s = Pair<XT>::dot(RZ_CVT_BF16(o0, 3), xp[3], s);
    s = Pair<XT>::dot(RZ_CVT_BF16(o1, 0), xp[4], s);
    s = Pair<XT>::dot(RZ_CVT_BF16(o1, 1), xp[5], s);
    s = Pair<XT>::dot(RZ_CVT_BF16(o1, 2), xp[6], s);
    s = Pair<XT>::dot(RZ_CVT_BF16(o1, 3), xp[7], s);
  }
}

// UNIT = 16-element blocks per lane step (2 when K % 32 == 0, else 1).
template <typename XT, int KIND, typename OT, int UNIT>
__global__ __launch_bounds__(256) void gemv_kernel(const XT* __restrict__ x,
                                                   const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scales,
                                                   const float* __restrict__ ts, int64_t n,
                                                   int64_t k, float m0, float m1,
                                                   OT* __restrict__ y) {
  typedef typename Pair<XT>::T P;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float2* lut = (float2*)smem;
  P* xs = (P*)(smem + 256 * sizeof(float2));
  {
    const uint32_t i = threadIdx.x;  // 256 threads, 256 scale bytes
    const float sb = scale_of_byte<KIND>(i);
    lut[i] = make_float2(sb, sb * special_of_byte<KIND>(i, m0, m1) * 0.5f);
  }
  for (int64_t i = threadIdx.x; i < k / 8; i += 256) ((uint4*)xs)[i] = ((const uint4*)x)[i];
  __syncthreads();

  const float st = *ts;
  const int lane = threadIdx.x & 63;
  const int64_t nchunk = k / (16 * UNIT);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); row < n; row += nwaves) {
    const uint8_t* crow = codes + row * (k / 2);
    const uint8_t* srow = scales + row * (k / 16);
    float acc = 0.0f;
    for (int64_t c = lane; c < nchunk; c += 64) {
      if constexpr (UNIT == 2) {
        const uint4 cw = load_nt16(crow + 16 * c);
        const uint32_t sw = *(const uint16_t*)(srow + 2 * c);
        const P* xp = xs + 16 * c;
        float d, s;
        block_dot<XT>(cw.x, cw.y, xp, d, s);
        float2 f = lut[sw & 0xFFu];
        acc = fmaf(d, f.x, acc);
        acc = fmaf(s, f.y, acc);
        block_dot<XT>(cw.z, cw.w, xp + 8, d, s);
        f = lut[sw >> 8];
        acc = fmaf(d, f.x, acc);
        acc = fmaf(s, f.y, acc);
      } else {
        const uint2 cw = load_nt8(crow + 8 * c);
        const uint32_t sw = srow[c];
        float d, s;
        block_dot<XT>(cw.x, cw.y, xs + 8 * c, d, s);
        const float2 f = lut[sw];
        acc = fmaf(d, f.x, acc);
        acc = fmaf(s, f.y, acc);
      }
    }
    acc = wave_sum_f32(acc);
    if (lane == 0) y[row] = gemv_out<OT>(acc * st);
  }
}

size_t gemv_ws_bytes(int64_t, int64_t) { return 0; }

template <typename XT, int KIND, typename OT>
static hipError_t run_gemv(const XT* x, const PackedView& w, OT* y, hipStream_t stream) {
  const int64_t n = w.rows, k = w.cols;
  const float m0 = 6.0f + 0.5f * (float)w.off_half[0];
  const float m1 = 6.0f + 0.5f * (float)w.off_half[KIND == kWeight ? 1 : 0];
  const size_t lds = 256 * sizeof(float2) + (size_t)k * 2;
  int64_t g = (n + 3) / 4;
  const int64_t cap = (int64_t)device_cu_count() * 4;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  if (k % 32 == 0) {
    auto kern = gemv_kernel<XT, KIND, OT, 2>;
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)g), dim3(256), lds, stream, x, w.codes, w.scales,
                       w.tensor_scale, n, k, m0, m1, y);
  } else {
    auto kern = gemv_kernel<XT, KIND, OT, 1>;
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)g), dim3(256), lds, stream, x, w.codes, w.scales,
                       w.tensor_scale, n, k, m0, m1, y);
  }
  return hipGetLastError();
}

template <typename XT, int KIND>
static hipError_t gemv_out_dispatch(const XT* x, const PackedView& w, void* y, int y_dtype,
                                    hipStream_t stream) {
  if (y_dtype == kF32) return run_gemv<XT, KIND>(x, w, (float*)y, stream);
  if (y_dtype == kF16) return run_gemv<XT, KIND>(x, w, (_Float16*)y, stream);
  return run_gemv<XT, KIND>(x, w, (__bf16*)y, stream);
}

hipError_t launch_gemv(const void* x, int x_dtype, const PackedView& w, void* y, int y_dtype,
                       void*, size_t, hipStream_t stream) {
  if (x_dtype == kF16) {
    if (w.kind == kWeight) return gemv_out_dispatch<_Float16, kWeight>((const _Float16*)x, w, y, y_dtype, stream);
    return gemv_out_dispatch<_Float16, kAct>((const _Float16*)x, w, y, y_dtype, stream);
  }
  if (w.kind == kWeight) return gemv_out_dispatch<__bf16, kWeight>((const __bf16*)x, w, y, y_dtype, stream);
  return gemv_out_dispatch<__bf16, kAct>((const __bf16*)x, w, y, y_dtype, stream);
}

}  // namespace rz
