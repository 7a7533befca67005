// rz_device.h -- device-side helpers shared by the librazer kernels (gfx950).
//
// Format facts used here come from "RaZeR: Pushing the Limits of NVFP4
// Quantization with Redundant Zero Remapping" (papernotes.org notes), Key
// designs 1-3: FP4-E2M1 elements {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign bit,
// 16-element blocks, an E3M3 (weights) or E4M3 (activations) block scale whose
// free bits hold the special-value selection, and special values
// sign * (6 + offset) with offsets in [-3.5, 3.5], step 0.5.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rz {

constexpr int kWave = 64;     // CDNA wavefront width
constexpr int kBlockElems = 16;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

enum Kind { kWeight = 0, kAct = 1 };
enum Dtype { kF32 = 0, kF16 = 1, kBF16 = 2 };

__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// Streaming (non-temporal) loads for data read exactly once.
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_nt8(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load((const u32x2_t*)p);
  return make_uint2(v.x, v.y);
}

// ---- wave reductions (64 lanes) ----------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Order one wave's LDS writes before its later LDS reads of data written by
// other lanes of the same wave (and those reads before the next writes).  The
// LDS executes one wave's operations in issue order, so only the compiler has
// to be kept from reordering them; it reasons per lane and would otherwise
// move a read above a write it sees as independent.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- block scale decode ------------------------------------------------------
// E3M3 (weights): 3 exponent bits, bias 3, 3 mantissa bits, subnormals, max 30.
// E4M3 (activations): OCP E4M3FN, bias 7, max 448.  The metadata bits of the
// scale byte are stripped by the mask.
template <int KIND>
__device__ __forceinline__ float scale_of_byte(uint32_t byte) {
  if (KIND == kWeight) {
    uint32_t c = byte & 0x3Fu;
    int e = (int)(c >> 3), m = (int)(c & 7u);
    return e ? __builtin_ldexpf((float)(8 + m), e - 6) : __builtin_ldexpf((float)m, -5);
  } else {
    uint32_t c = byte & 0x7Fu;
    int e = (int)(c >> 3), m = (int)(c & 7u);
    return e ? __builtin_ldexpf((float)(8 + m), e - 10) : __builtin_ldexpf((float)m, -9);
  }
}

// Special value selected by a scale byte: bit 7 = sign, bit 6 = pair (weights).
template <int KIND>
__device__ __forceinline__ float special_of_byte(uint32_t byte, float m0, float m1) {
  float mag = (KIND == kWeight && (byte & 0x40u)) ? m1 : m0;
  return (byte & 0x80u) ? -mag : mag;
}

// Group-scale variant: an FP16 block scale whose sign bit and top exponent bit
// carry the metadata (sign of the special value, pair); the other 14 bits are
// the scale, an FP16 number with exponent field 0..15.
constexpr float kF16ScaleMax = 1.9990234375f;  // 14-bit code 0x3FFF
__device__ __forceinline__ float scale_of_f16word(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0x3FFFu));
}
__device__ __forceinline__ float special_of_f16word(uint32_t w, float m0, float m1) {
  float mag = (w & 0x4000u) ? m1 : m0;
  return (w & 0x8000u) ? -mag : mag;
}

// FP4-E2M1 magnitude of a 3-bit magnitude field, times 2 (an integer):
// {0, 1, 2, 3, 4, 6, 8, 12} packed as nibbles.
__device__ __forceinline__ uint32_t fp4_mag_x2(uint32_t m) { return (0xC8643210u >> (4u * m)) & 15u; }

// ---- packed-nibble helpers ---------------------------------------------------
// For a dword of 8 codes, returns the same dword with nibble 0b0100 (FP4 +2.0)
// where the code is the remapped 0b1000 and 0 elsewhere.  (c & 7) + 7 sets bit 3
// of a nibble unless its magnitude is zero; no carry crosses nibbles.
__device__ __forceinline__ uint32_t special_onehot_x2(uint32_t c) {
  uint32_t u = (c & 0x77777777u) + 0x77777777u;
  return ((~u & c) & 0x88888888u) >> 1;
}

}  // namespace rz
