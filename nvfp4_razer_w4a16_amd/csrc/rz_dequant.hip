// rz_dequant.hip -- RaZeR decoder for gfx950 (streaming, eight elements per lane and step).
//
// "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
// Remapping" (papernotes.org notes), Key design 3 and the complete example:
// the decoder reads the block's metadata bits, forms 6 + offset for the chosen
// pair, attaches the sign and emits that value wherever the remapped -0 code
// appears; all other codes are plain FP4.  Output = value * sb * st, computed
// as fl32(fl32(value * sb) * st) (value * sb has at most 9 significant bits, so
// the first product is exact) and, for 16-bit outputs, rounded to nearest even.
#include "rz_device.h"
#include "rz_launch.h"

namespace rz {

template <typename OT> __device__ __forceinline__ OT to_out(float v);
template <> __device__ __forceinline__ float to_out<float>(float v) { return v; }
template <> __device__ __forceinline__ _Float16 to_out<_Float16>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ __bf16 to_out<__bf16>(float v) { return (__bf16)v; }

// Eight elements (one code dword, half a block) per lane and step, so each
// wave's loads and stores are contiguous: 256 code bytes in, 1 KiB (16-bit)
// or 2 KiB (fp32) out.  The gfx950 packed FP4 conversion gives the exact
// values, with -0 for the remapped code; that -0 is detected on the converted
// value before any scaling, so an underflowing product can never pass for it.
template <typename OT> struct Out8;
template <> struct Out8<float> {
  static __device__ __forceinline__ void store(float* o, const float (&v)[8]) {
    ((float4*)o)[0] = make_float4(v[0], v[1], v[2], v[3]);
    ((float4*)o)[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
};
template <typename OT> struct Out8 {
  static __device__ __forceinline__ void store(OT* o, const float (&v)[8]) {
    OT h[8];
#pragma unroll
    for (int j = 0; j < 8; j++) h[j] = to_out<OT>(v[j]);
    *(uint4*)o = *(const uint4*)h;
  }
};

constexpr int kDqUnroll = 4;  // code dwords in flight per lane

template <int KIND, typename OT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ ts, int64_t ndw,
                                                      float m0, float m1, OT* __restrict__ out) {
  const float st = ts ? *ts : 1.0f;  // no tensor scale: value * sb
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t d0 = (int64_t)blockIdx.x * 256 + threadIdx.x; d0 < ndw; d0 += kDqUnroll * stride) {
    uint32_t w[kDqUnroll], sbyte[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; u++) {
      const int64_t d = d0 + u * stride;
      w[u] = d < ndw ? codes[d] : 0u;
      sbyte[u] = d < ndw ? scales[d >> 1] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kDqUnroll; u++) {
      const int64_t d = d0 + u * stride;
      if (d >= ndw) break;
      const float sb = scale_of_byte<KIND>(sbyte[u]);
      const float svt = (special_of_byte<KIND>(sbyte[u], m0, m1) * sb) * st;
      float v[8];
#pragma unroll
      for (int p = 0; p < 4; p++) {
        float2_t f;
        switch (p) {
          case 0: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 0); break;
          case 1: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 1); break;
          case 2: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 2); break;
          default: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[u], 1.0f, 3); break;
        }
        // The halves pass through an empty asm before the -0 tests: without
        // it this compiler folds the two tests of one conversion into one.
        float f0 = f[0], f1 = f[1];
        asm volatile("" : "+v"(f0), "+v"(f1));
        v[2 * p] = __builtin_bit_cast(uint32_t, f0) == 0x80000000u ? svt : (f0 * sb) * st;
        v[2 * p + 1] = __builtin_bit_cast(uint32_t, f1) == 0x80000000u ? svt : (f1 * sb) * st;
      }
      Out8<OT>::store(out + 8 * d, v);
    }
  }
}

// Block-size and scale-format variants (blocks of 16 << (blog2 - 4) elements,
// byte or FP16 group scales): one code dword per lane and step, its block's
// scale word read directly; the same value rule and fp32 operation order.
template <int KIND, typename OT>
__global__ __launch_bounds__(256) void dequant_variant_kernel(const uint32_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales,
                                                              const float* __restrict__ ts, int64_t ndw,
                                                              float m0, float m1, int blog2, int sfmt,
                                                              OT* __restrict__ out) {
  const float st = ts ? *ts : 1.0f;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x; d < ndw; d += stride) {
    const uint32_t w = codes[d];
    const int64_t blk = (8 * d) >> blog2;
    const uint32_t sw = sfmt ? (uint32_t)((const uint16_t*)scales)[blk] : (uint32_t)scales[blk];
    const float sb = sfmt ? scale_of_f16word(sw) : scale_of_byte<KIND>(sw);
    const float sv = sfmt ? special_of_f16word(sw, m0, m1) : special_of_byte<KIND>(sw, m0, m1);
    const float svt = (sv * sb) * st;
    float v[8];
#pragma unroll
    for (int p = 0; p < 4; p++) {
      float2_t f;
      switch (p) {
        case 0: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
        case 1: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
        case 2: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
        default: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
      }
      float f0 = f[0], f1 = f[1];
      asm volatile("" : "+v"(f0), "+v"(f1));  // keeps the two -0 tests apart (see above)
      v[2 * p] = __builtin_bit_cast(uint32_t, f0) == 0x80000000u ? svt : (f0 * sb) * st;
      v[2 * p + 1] = __builtin_bit_cast(uint32_t, f1) == 0x80000000u ? svt : (f1 * sb) * st;
    }
    Out8<OT>::store(out + 8 * d, v);
  }
}

template <int KIND, typename OT>
static void run(const PackedView& t, OT* out, bool scaled, hipStream_t stream) {
  const int64_t ndw = t.rows * t.cols / 8;
  int64_t g = (ndw + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  const float m0 = 6.0f + 0.5f * (float)t.off_half[0];
  const float m1 = 6.0f + 0.5f * (float)t.off_half[KIND == kWeight ? 1 : 0];
  if (!default_layout(t))
    hipLaunchKernelGGL((dequant_variant_kernel<KIND, OT>), dim3((unsigned)g), dim3(256), 0, stream,
                       (const uint32_t*)t.codes, t.scales, scaled ? t.tensor_scale : nullptr, ndw, m0, m1,
                       t.blog2, t.sfmt, out);
  else
    hipLaunchKernelGGL((dequant_kernel<KIND, OT>), dim3((unsigned)g), dim3(256), 0, stream,
                       (const uint32_t*)t.codes, t.scales, scaled ? t.tensor_scale : nullptr, ndw, m0, m1, out);
}

static hipError_t dequant_dispatch(const PackedView& t, void* out, int out_dtype, bool scaled,
                                   hipStream_t stream) {
  if (t.kind == kWeight) {
    if (out_dtype == kF32) run<kWeight>(t, (float*)out, scaled, stream);
    else if (out_dtype == kF16) run<kWeight>(t, (_Float16*)out, scaled, stream);
    else run<kWeight>(t, (__bf16*)out, scaled, stream);
  } else {
    if (out_dtype == kF32) run<kAct>(t, (float*)out, scaled, stream);
    else if (out_dtype == kF16) run<kAct>(t, (_Float16*)out, scaled, stream);
    else run<kAct>(t, (__bf16*)out, scaled, stream);
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const PackedView& t, void* out, int out_dtype, hipStream_t stream) {
  return dequant_dispatch(t, out, out_dtype, true, stream);
}

// value * sb without the tensor scale: FP4 or special value (at most 5
// significant bits) times a 4-bit scale mantissa, exact in fp16.
hipError_t launch_dequant_unscaled(const PackedView& t, void* out, int out_dtype, hipStream_t stream) {
  return dequant_dispatch(t, out, out_dtype, false, stream);
}

}  // namespace rz
