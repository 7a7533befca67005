// rz_dequant.hip -- RaZeR decoder for gfx950 (streaming, one block per thread).
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

template <int KIND, typename OT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint2* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ ts, int64_t nblk,
                                                      float m0, float m1, OT* __restrict__ out) {
  const float st = *ts;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk; b += stride) {
    const uint2 cw = codes[b];
    const uint32_t sbyte = scales[b];
    const float sb = scale_of_byte<KIND>(sbyte);
    const float sv = special_of_byte<KIND>(sbyte, m0, m1) * sb;
    OT v[16];
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const uint32_t nib = ((j < 8 ? cw.x : cw.y) >> (4 * (j & 7))) & 15u;
      // |FP4| * 2 from the magnitude field, then halve: exact small integers.
      const float mag = (float)fp4_mag_x2(nib & 7u) * 0.5f;
      float val = (nib & 8u) ? -mag : mag;
      val = (nib == 8u) ? sv : val * sb;
      v[j] = to_out<OT>(val * st);
    }
    OT* o = out + 16 * b;
    if (sizeof(OT) == 4) {
#pragma unroll
      for (int i = 0; i < 4; i++) ((uint4*)o)[i] = ((uint4*)v)[i];
    } else {
#pragma unroll
      for (int i = 0; i < 2; i++) ((uint4*)o)[i] = ((uint4*)v)[i];
    }
  }
}

template <int KIND, typename OT>
static void run(const PackedView& t, OT* out, hipStream_t stream) {
  const int64_t nblk = t.rows * t.cols / 16;
  int64_t g = (nblk + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  const float m0 = 6.0f + 0.5f * (float)t.off_half[0];
  const float m1 = 6.0f + 0.5f * (float)t.off_half[KIND == kWeight ? 1 : 0];
  hipLaunchKernelGGL((dequant_kernel<KIND, OT>), dim3((unsigned)g), dim3(256), 0, stream,
                     (const uint2*)t.codes, t.scales, t.tensor_scale, nblk, m0, m1, out);
}

hipError_t launch_dequant(const PackedView& t, void* out, int out_dtype, hipStream_t stream) {
  if (t.kind == kWeight) {
    if (out_dtype == kF32) run<kWeight>(t, (float*)out, stream);
    else if (out_dtype == kF16) run<kWeight>(t, (_Float16*)out, stream);
    else run<kWeight>(t, (__bf16*)out, stream);
  } else {
    if (out_dtype == kF32) run<kAct>(t, (float*)out, stream);
    else if (out_dtype == kF16) run<kAct>(t, (_Float16*)out, stream);
    else run<kAct>(t, (__bf16*)out, stream);
  }
  return hipGetLastError();
}

}  // namespace rz
