// rz_gemm.hip -- batched W4A16 product y[M, N] = x[M, K] * W^T on gfx950 MFMA.
//
// "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
// Remapping" (papernotes.org notes), Key design 3: weight-only GEMM kernels
// that decompress RaZeR weights inside the kernel; "Technical Summary: RaZeR
// ..." (gist.science), §2.3 and §4 (moderate and large batches).
//
// Each 256-thread workgroup owns a BM x BN output tile.  Per K step of BK
// elements, the x tile is copied to LDS and the weight tile is decoded once to
// 16-bit floats (value * block scale; the remapped -0 code becomes the block's
// special value) and written to LDS, so the four waves share one decode.  The
// waves then run v_mfma_f32_32x32x16 (bf16 or f16) on 64 x 64 sub-tiles with
// fp32 accumulators; the tensor scale is applied once in the epilogue.
#include "rz_device.h"
#include "rz_launch.h"

namespace rz {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

template <typename XT> struct Mfma32;
template <> struct Mfma32<__bf16> {
  typedef bf16x8_t V;
  static __device__ __forceinline__ floatx16 run(V a, V b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma32<_Float16> {
  typedef f16x8_t V;
  static __device__ __forceinline__ floatx16 run(V a, V b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return (__bf16)v; }

// Decode one 16-element block to value * sb in XT (exact for f16; bf16 rounds
// only special values with 5 significant bits times a 4-bit scale mantissa).
template <int KIND, typename XT>
__device__ __forceinline__ void decode_block(uint2 cw, uint32_t sbyte, float m0, float m1,
                                             XT (&out)[16]) {
  const float sb = scale_of_byte<KIND>(sbyte);
  const float sv = special_of_byte<KIND>(sbyte, m0, m1) * sb;
#pragma unroll
  for (int j = 0; j < 16; j++) {
    const uint32_t nib = ((j < 8 ? cw.x : cw.y) >> (4 * (j & 7))) & 15u;
    const float mag = (float)fp4_mag_x2(nib & 7u) * (0.5f * sb);
    const float val = (nib == 8u) ? sv : ((nib & 8u) ? -mag : mag);
    out[j] = from_f32<XT>(val);
  }
}

constexpr int kBM = 128, kBN = 128, kBK = 32, kLds = kBK + 8;

template <typename XT, int KIND, typename OT>
__global__ __launch_bounds__(256) void gemm_kernel(const XT* __restrict__ x, int64_t m,
                                                   const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scales,
                                                   const float* __restrict__ ts, int64_t n,
                                                   int64_t k, float m0, float m1,
                                                   OT* __restrict__ y) {
  typedef typename Mfma32<XT>::V V;
  __shared__ __attribute__((aligned(16))) XT As[kBM * kLds];
  __shared__ __attribute__((aligned(16))) XT Bs[kBN * kLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m_base = (int64_t)blockIdx.y * kBM, n_base = (int64_t)blockIdx.x * kBN;
  const int64_t kblocks = k / 16;
  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  const int r = tid >> 1, h = tid & 1;
  for (int64_t kb0 = 0; kb0 < kblocks; kb0 += 2) {
    const int64_t kb = kb0 + h;
    {  // x tile: row r, block h
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
      const int64_t gr = m_base + r;
      if (gr < m && kb < kblocks) {
        const uint4* p = (const uint4*)(x + gr * k + kb * 16);
        v0 = p[0];
        v1 = p[1];
      }
      uint4* d = (uint4*)(As + r * kLds + h * 16);
      d[0] = v0;
      d[1] = v1;
    }
    {  // weight tile: weight row r, block h, decoded once
      XT vals[16];
      const int64_t gn = n_base + r;
      if (gn < n && kb < kblocks) {
        const uint2 cw = *(const uint2*)(codes + gn * (k / 2) + kb * 8);
        const uint32_t sbyte = scales[gn * (k / 16) + kb];
        decode_block<KIND, XT>(cw, sbyte, m0, m1, vals);
      } else {
#pragma unroll
        for (int j = 0; j < 16; j++) vals[j] = from_f32<XT>(0.0f);
      }
      uint4* d = (uint4*)(Bs + r * kLds + h * 16);
      d[0] = ((uint4*)vals)[0];
      d[1] = ((uint4*)vals)[1];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      V a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; i++)
        a[i] = *(const V*)(As + (wm * 64 + i * 32 + (lane & 31)) * kLds + kk + 8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 2; j++)
        b[j] = *(const V*)(Bs + (wn * 64 + j * 32 + (lane & 31)) * kLds + kk + 8 * (lane >> 5));
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = Mfma32<XT>::run(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  const float st = *ts;
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int64_t gr = m_base + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int64_t gc = n_base + wn * 64 + j * 32 + (lane & 31);
        if (gr < m && gc < n) y[gr * n + gc] = from_f32<OT>(acc[i][j][e] * st);
      }
}

// ---- large tiles: 256 x 256 x 64, double-buffered LDS, register prefetch -------
//
// For M >= 256 (prefill).  Four waves, each owning a 128 x 128 sub-tile (4 x 4
// MFMA 32x32x16 tiles, 256 fp32 accumulators per lane).  Per K step each
// thread prefetches 128 bytes of x and one weight row's 32 code bytes + 4
// scale bytes into registers while the waves run the step's 64 MFMAs; then
// it writes the x bytes and the decoded weight row (64 values) into the other
// LDS buffer.  LDS rows are padded by 16 bytes so the 16-byte fragment reads
// of 32 consecutive rows hit distinct banks.
//
// Decode (per pair of codes): the packed FP4 conversion, an exact multiply by
// sb, and a bit select that puts the block's SV * sb where the remapped code
// (converted to -0) sits; see decode_pair_impl.
constexpr int kTM = 256, kTN = 256, kTK = 64, kTS = kTK + 8;

typedef short short2_t __attribute__((ext_vector_type(2)));
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

template <typename XT> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<__bf16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){a, b}, bf162_t));
}
template <> __device__ __forceinline__ uint32_t pack2<_Float16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, (half2_t){(_Float16)a, (_Float16)b});
}
template <typename XT> __device__ __forceinline__ uint32_t bits16(float v);
template <> __device__ __forceinline__ uint32_t bits16<__bf16>(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v);
}
template <> __device__ __forceinline__ uint32_t bits16<_Float16>(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}

// Two codes (byte SEL of w) -> one packed 16-bit pair of value * sb, with the
// remapped code replaced by svb2 (SV * sb in both halves).  The remapped code
// converts to -0; it is detected on the unscaled pair (the int16 minimum:
// max_i16(p, 0x8001) ^ p is 1 there and 0 elsewhere, negated into a 0xFFFF
// mask) so no later rounding step can touch the sign of that zero.
__device__ __forceinline__ uint32_t remapped_mask(uint32_t p) {
  const short2_t q = __builtin_elementwise_max(__builtin_bit_cast(short2_t, p),
                                               (short2_t){(short)0x8001, (short)0x8001});
  const ushort2_t one = __builtin_bit_cast(ushort2_t, __builtin_bit_cast(uint32_t, q) ^ p);
  return __builtin_bit_cast(uint32_t, (ushort2_t){0, 0} - one);
}

// fp16: FP4 -> f16 pair directly, then an exact packed multiply by sb (value *
// sb has at most 9 significant bits).
template <typename XT, int SEL>
__device__ __forceinline__ uint32_t decode_pair_impl(uint32_t w, float sb, uint32_t svb2) {
  if constexpr (__is_same(XT, _Float16)) {
    const half2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
    const uint32_t mask = remapped_mask(__builtin_bit_cast(uint32_t, h));
    const _Float16 s16 = (_Float16)sb;  // exact: sb has 4 significant bits, in fp16 range
    const uint32_t v = __builtin_bit_cast(uint32_t, h * (half2_t){s16, s16});
    return (mask & svb2) | (~mask & v);
  } else {
    // bf16: FP4 -> fp32 pair, scaled with fma(f, sb, -0) so a -0 stays -0,
    // then rounded to bf16 (exact unless an SV has 5 significant bits).
    const float2_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
    const uint32_t p = pack2<XT>(__builtin_fmaf(f[0], sb, -0.0f), __builtin_fmaf(f[1], sb, -0.0f));
    const uint32_t mask = remapped_mask(p);
    return (mask & svb2) | (~mask & p);
  }
}

template <typename XT, int KIND>
__device__ __forceinline__ void decode_row64(const uint4 (&c)[2], uint32_t sw, float m0, float m1,
                                             uint4 (&out)[8]) {
#pragma unroll
  for (int blk = 0; blk < 4; blk++) {
    const uint32_t byte = (sw >> (8 * blk)) & 0xFFu;
    const float sb = scale_of_byte<KIND>(byte);
    const uint32_t svb = bits16<XT>(special_of_byte<KIND>(byte, m0, m1) * sb);
    const uint32_t svb2 = svb | (svb << 16);
    const uint4 cw = c[blk >> 1];
    const uint32_t w0 = (blk & 1) ? cw.z : cw.x;
    const uint32_t w1 = (blk & 1) ? cw.w : cw.y;
    out[2 * blk] = make_uint4(decode_pair_impl<XT, 0>(w0, sb, svb2), decode_pair_impl<XT, 1>(w0, sb, svb2),
                              decode_pair_impl<XT, 2>(w0, sb, svb2), decode_pair_impl<XT, 3>(w0, sb, svb2));
    out[2 * blk + 1] = make_uint4(decode_pair_impl<XT, 0>(w1, sb, svb2), decode_pair_impl<XT, 1>(w1, sb, svb2),
                                  decode_pair_impl<XT, 2>(w1, sb, svb2), decode_pair_impl<XT, 3>(w1, sb, svb2));
  }
}

template <typename XT, int KIND, typename OT>
__global__ __launch_bounds__(256) void gemm_tile256_kernel(const XT* __restrict__ x, int64_t m,
                                                           const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ ts, int64_t n,
                                                           int64_t k, float m0, float m1,
                                                           OT* __restrict__ y) {
  typedef typename Mfma32<XT>::V V;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  XT* As = (XT*)smem;                    // [2][kTM * kTS]
  XT* Bs = As + 2 * kTM * kTS;           // [2][kTN * kTS]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t ntn = (n + kTN - 1) / kTN;
  const int64_t m_base = (int64_t)(blockIdx.x / ntn) * kTM;
  const int64_t n_base = (int64_t)(blockIdx.x % ntn) * kTN;
  const int ktiles = (int)(k / kTK);

  uint4 areg[8];
  uint4 creg[2];
  uint32_t sreg;
  const int64_t gn = n_base + tid;
  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kTK;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int idx = i * 256 + tid;
      const int64_t gr = m_base + (idx >> 3);
      areg[i] = gr < m ? *(const uint4*)(x + gr * k + k0 + (idx & 7) * 8) : make_uint4(0, 0, 0, 0);
    }
    if (gn < n) {
      const uint4* cp = (const uint4*)(codes + gn * (k / 2) + k0 / 2);
      creg[0] = cp[0];
      creg[1] = cp[1];
      sreg = *(const uint32_t*)(scales + gn * (k / 16) + k0 / 16);
    } else {
      creg[0] = creg[1] = make_uint4(0, 0, 0, 0);
      sreg = 0;
    }
  };
  auto lstore = [&](int buf) {
    XT* a = As + buf * kTM * kTS;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int idx = i * 256 + tid;
      *(uint4*)(a + (idx >> 3) * kTS + (idx & 7) * 8) = areg[i];
    }
    uint4 dec[8];
    decode_row64<XT, KIND>(creg, sreg, m0, m1, dec);
    uint4* b = (uint4*)(Bs + buf * kTN * kTS + tid * kTS);
#pragma unroll
    for (int i = 0; i < 8; i++) b[i] = dec[i];
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < ktiles; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < ktiles) gload(kt + 1);
    const XT* a = As + cur * kTM * kTS;
    const XT* b = Bs + cur * kTN * kTS;
#pragma unroll
    for (int kk = 0; kk < kTK; kk += 16) {
      V av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        av[i] = *(const V*)(a + (wm * 128 + i * 32 + (lane & 31)) * kTS + kk + 8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 4; j++)
        bv[j] = *(const V*)(b + (wn * 128 + j * 32 + (lane & 31)) * kTS + kk + 8 * (lane >> 5));
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = Mfma32<XT>::run(av[i], bv[j], acc[i][j]);
    }
    if (kt + 1 < ktiles) lstore(cur ^ 1);
    __syncthreads();
  }

  const float st = *ts;
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t gc = n_base + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int64_t gr = m_base + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (gr < m && gc < n) y[gr * n + gc] = from_f32<OT>(acc[i][j][e] * st);
      }
    }
}

size_t gemm_ws_bytes(int64_t, int64_t, int64_t) { return 0; }

template <typename XT, int KIND, typename OT>
static hipError_t run_gemm(const XT* x, int64_t m, const PackedView& w, OT* y,
                           hipStream_t stream) {
  const int64_t n = w.rows, k = w.cols;
  const float m0 = 6.0f + 0.5f * (float)w.off_half[0];
  const float m1 = 6.0f + 0.5f * (float)w.off_half[KIND == kWeight ? 1 : 0];
  if (m >= kTM && k % kTK == 0) {
    auto kern = gemm_tile256_kernel<XT, KIND, OT>;
    const size_t lds = (size_t)2 * (kTM + kTN) * kTS * sizeof(XT);
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int64_t tiles = ((m + kTM - 1) / kTM) * ((n + kTN - 1) / kTN);
    hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(256), lds, stream, x, m, w.codes,
                       w.scales, w.tensor_scale, n, k, m0, m1, y);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
  hipLaunchKernelGGL((gemm_kernel<XT, KIND, OT>), grid, dim3(256), 0, stream, x, m, w.codes,
                     w.scales, w.tensor_scale, n, k, m0, m1, y);
  return hipGetLastError();
}

template <typename XT, int KIND>
static hipError_t gemm_out_dispatch(const XT* x, int64_t m, const PackedView& w, void* y,
                                    int y_dtype, hipStream_t stream) {
  if (y_dtype == kF32) return run_gemm<XT, KIND>(x, m, w, (float*)y, stream);
  if (y_dtype == kF16) return run_gemm<XT, KIND>(x, m, w, (_Float16*)y, stream);
  return run_gemm<XT, KIND>(x, m, w, (__bf16*)y, stream);
}

hipError_t launch_gemm(const void* x, int x_dtype, int64_t m, const PackedView& w, void* y,
                       int y_dtype, void*, size_t, hipStream_t stream) {
  if (x_dtype == kF16) {
    if (w.kind == kWeight) return gemm_out_dispatch<_Float16, kWeight>((const _Float16*)x, m, w, y, y_dtype, stream);
    return gemm_out_dispatch<_Float16, kAct>((const _Float16*)x, m, w, y, y_dtype, stream);
  }
  if (w.kind == kWeight) return gemm_out_dispatch<__bf16, kWeight>((const __bf16*)x, m, w, y, y_dtype, stream);
  return gemm_out_dispatch<__bf16, kAct>((const __bf16*)x, m, w, y, y_dtype, stream);
}

}  // namespace rz
