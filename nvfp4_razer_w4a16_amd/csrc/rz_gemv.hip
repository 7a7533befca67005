// rz_gemv.hip -- batch-1 W4A16 product y = x * W^T on gfx950, decoding the
// RaZeR weight format in registers.
//
// "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
// Remapping" (papernotes.org notes), Key design 3: weight-only GEMV kernels
// decode the packed weights inside the kernel, and the launch is sized so
// small matrices are not over-split; "Technical Summary: RaZeR ..."
// (gist.science), §2.3.  The pages' kernel (group-128 FP16 scales on another
// GPU) is prior art only; this one is written for CDNA4:
//   - a wavefront owns R weight rows; lane l takes chunks (32 or 16 elements)
//     l, l+64, ..., so every 16-byte code load is one coalesced 1 KiB wave
//     access, and all R * CPL chunk loads of a pass are issued before any is
//     consumed (and before x is staged), keeping enough bytes in flight to
//     cover HBM latency;
//   - x is staged once per workgroup in LDS (zero padded), with a 256-entry
//     table of (sb, sb * SV / 2) indexed by the scale byte;
//   - codes become fp16/bf16 pairs with the gfx950 packed FP4 conversion and
//     are contracted with x by v_dot2 (fp32 accumulate).  The remapped code
//     0b1000 converts to -0 (0x8000), the only pair half below -0.25 when read
//     as int16, so a packed int16 max against -0.25 followed by an xor with
//     the converted pair leaves exactly 0.25 at remapped positions and 0
//     elsewhere; a second v_dot2 of that one-hot with x gives sum(x) / 4 over
//     the remapped positions, and the block sum is
//     dot * sb + onehot_dot * (sb * SV * 4);
//   - each row's 64 lane partials are summed across the wave and scaled once
//     by the tensor scale.
#include "rz_device.h"
#include "rz_launch.h"

namespace rz {

typedef short short2_t __attribute__((ext_vector_type(2)));

template <typename XT> struct Pair;
template <> struct Pair<_Float16> {
  typedef half2_t T;
  static constexpr short kQuarterNeg = (short)0xB400;  // -0.25 in fp16
  template <int SEL> static __device__ __forceinline__ T cvt(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
  }
  static __device__ __forceinline__ float dot(T a, T b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
  }
};
template <> struct Pair<__bf16> {
  typedef bf162_t T;
  static constexpr short kQuarterNeg = (short)0xBE80;  // -0.25 in bf16
  template <int SEL> static __device__ __forceinline__ T cvt(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
  }
  static __device__ __forceinline__ float dot(T a, T b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
};

// 0.25 where the converted half is the remapped -0, 0 elsewhere.  Every other
// converted half (+0, +/-0.5 .. +/-6) is >= -0.5 > -0.25 - as int16 patterns
// it compares above the -0.25 pattern, which compares above 0x8000.
template <typename XT>
__device__ __forceinline__ typename Pair<XT>::T remapped_onehot(typename Pair<XT>::T p) {
  const short2_t q = __builtin_elementwise_max(__builtin_bit_cast(short2_t, p),
                                               (short2_t){Pair<XT>::kQuarterNeg, Pair<XT>::kQuarterNeg});
  return __builtin_bit_cast(typename Pair<XT>::T,
                            __builtin_bit_cast(uint32_t, q) ^ __builtin_bit_cast(uint32_t, p));
}

// Contract 8 codes (one dword; byte j holds elements 2j, 2j+1, low nibble
// first) with 4 x pairs: d += FP4 dot, s += one-hot dot.
template <typename XT, int SEL>
__device__ __forceinline__ void dot2_step(uint32_t w, typename Pair<XT>::T xv, float& d, float& s) {
  const typename Pair<XT>::T p = Pair<XT>::template cvt<SEL>(w);
  d = Pair<XT>::dot(p, xv, d);
  s = Pair<XT>::dot(remapped_onehot<XT>(p), xv, s);
}

// One 16-element block (codes w0: elements 0..7, w1: 8..15).
template <typename XT>
__device__ __forceinline__ void block_dot(uint32_t w0, uint32_t w1, const typename Pair<XT>::T* xp,
                                          float& d, float& s) {
  d = 0.0f;
  s = 0.0f;
  dot2_step<XT, 0>(w0, xp[0], d, s);
  dot2_step<XT, 1>(w0, xp[1], d, s);
  dot2_step<XT, 2>(w0, xp[2], d, s);
  dot2_step<XT, 3>(w0, xp[3], d, s);
  dot2_step<XT, 0>(w1, xp[4], d, s);
  dot2_step<XT, 1>(w1, xp[5], d, s);
  dot2_step<XT, 2>(w1, xp[6], d, s);
  dot2_step<XT, 3>(w1, xp[7], d, s);
}

struct GemvArgs {
  const void* x;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* ts;
  void* y;
  int64_t n, k, nchunk;
  int npass, kind, ydt;
  float m0, m1;
};

__device__ __forceinline__ void store_out(void* y, int64_t i, float v, int ydt) {
  if (ydt == kF32) ((float*)y)[i] = v;
  else if (ydt == kF16) ((_Float16*)y)[i] = (_Float16)v;
  else ((__bf16*)y)[i] = (__bf16)v;
}

template <int UNIT> struct Chunk;
template <> struct Chunk<2> {  // 32 elements: 16 code bytes, 2 scale bytes
  uint4 c;
  uint32_t s;
  __device__ __forceinline__ void load(const uint8_t* crow, const uint8_t* srow, int64_t i) {
    c = load_nt16(crow + 16 * i);
    s = *(const uint16_t*)(srow + 2 * i);
  }
  __device__ __forceinline__ void zero() { c = make_uint4(0, 0, 0, 0); s = 0; }
  __device__ __forceinline__ uint32_t w(int j) const { return j == 0 ? c.x : j == 1 ? c.y : j == 2 ? c.z : c.w; }
};
template <> struct Chunk<1> {  // 16 elements: 8 code bytes, 1 scale byte
  uint2 c;
  uint32_t s;
  __device__ __forceinline__ void load(const uint8_t* crow, const uint8_t* srow, int64_t i) {
    c = load_nt8(crow + 8 * i);
    s = srow[i];
  }
  __device__ __forceinline__ void zero() { c = make_uint2(0, 0); s = 0; }
  __device__ __forceinline__ uint32_t w(int j) const { return j == 0 ? c.x : c.y; }
};

// R rows per wave, CPL chunks per lane per pass, UNIT blocks per chunk.
template <typename XT, int UNIT, int R, int CPL>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  typedef typename Pair<XT>::T P;
  constexpr int kPairsPerChunk = 8 * UNIT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float2* lut = (float2*)smem;
  P* xs = (P*)(smem + 256 * sizeof(float2));

  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  const int64_t rcb = a.k / 2, rsb = a.k / 16;

  Chunk<UNIT> ch[R][CPL];
  auto load_pass = [&](int p) {
#pragma unroll
    for (int r = 0; r < R; r++) {
      const int64_t row = row0 + r;
      const uint8_t* crow = a.codes + row * rcb;
      const uint8_t* srow = a.scales + row * rsb;
#pragma unroll
      for (int i = 0; i < CPL; i++) {
        const int64_t c = ((int64_t)p * CPL + i) * 64 + lane;
        if (row < a.n && c < a.nchunk) ch[r][i].load(crow, srow, c);
        else ch[r][i].zero();
      }
    }
  };
  load_pass(0);  // weight bytes in flight while x is staged

  {
    const uint32_t i = threadIdx.x;
    float sb, sv;
    if (a.kind == kWeight) {
      sb = scale_of_byte<kWeight>(i);
      sv = special_of_byte<kWeight>(i, a.m0, a.m1);
    } else {
      sb = scale_of_byte<kAct>(i);
      sv = special_of_byte<kAct>(i, a.m0, a.m1);
    }
    lut[i] = make_float2(sb, sb * sv * 4.0f);
  }
  const int64_t xvec = a.k / 8;                                           // 16-byte x vectors
  const int64_t xpad = (int64_t)a.npass * CPL * 64 * kPairsPerChunk / 4;  // padded, in vectors
  const uint4* xg = (const uint4*)a.x;
  for (int64_t i = threadIdx.x; i < xpad; i += 256)
    ((uint4*)xs)[i] = i < xvec ? xg[i] : make_uint4(0, 0, 0, 0);
  __syncthreads();

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; r++) acc[r] = 0.0f;
  for (int p = 0; p < a.npass; p++) {
    if (p > 0) load_pass(p);
#pragma unroll
    for (int i = 0; i < CPL; i++) {
      const int64_t c = ((int64_t)p * CPL + i) * 64 + lane;
      P xv[kPairsPerChunk];
#pragma unroll
      for (int q = 0; q < kPairsPerChunk / 4; q++)
        ((uint4*)xv)[q] = ((const uint4*)(xs + c * kPairsPerChunk))[q];
#pragma unroll
      for (int r = 0; r < R; r++) {
#pragma unroll
        for (int u = 0; u < UNIT; u++) {
          float d, s;
          block_dot<XT>(ch[r][i].w(2 * u), ch[r][i].w(2 * u + 1), xv + 8 * u, d, s);
          const float2 f = lut[(ch[r][i].s >> (8 * u)) & 0xFFu];
          acc[r] = fmaf(d, f.x, acc[r]);
          acc[r] = fmaf(s, f.y, acc[r]);
        }
      }
    }
  }

  const float st = *a.ts;
#pragma unroll
  for (int r = 0; r < R; r++) {
    const float v = wave_sum_f32(acc[r]);
    if (lane == r && row0 + r < a.n) store_out(a.y, row0 + r, v * st, a.ydt);
  }
}

size_t gemv_ws_bytes(int64_t, int64_t) { return 0; }

template <typename XT, int UNIT, int R, int CPL>
static hipError_t launch_cfg(const GemvArgs& a, hipStream_t stream) {
  constexpr int kPairsPerChunk = 8 * UNIT;
  const size_t lds = 256 * sizeof(float2) + (size_t)a.npass * CPL * 64 * kPairsPerChunk * 4;
  auto kern = gemv_kernel<XT, UNIT, R, CPL>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t waves = (a.n + R - 1) / R;
  const int64_t grid = (waves + 3) / 4;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, stream, a);
  return hipGetLastError();
}

// Launch sizing (the CDNA counterpart of the pages' SM-launch trimming): pick
// chunks per lane so one pass covers K where possible, then the largest row
// group R that still leaves >= 6 waves per SIMD for latency hiding.
template <typename XT, int UNIT>
static hipError_t dispatch(GemvArgs a, hipStream_t stream) {
  const int64_t per_lane = (a.nchunk + 63) / 64;
  const int cpl = per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : per_lane <= 7 ? 7 : 8;
  a.npass = (int)((a.nchunk + 64LL * cpl - 1) / (64LL * cpl));
  if (a.npass < 1) a.npass = 1;
  const int64_t simds = 4LL * device_cu_count();
  int r = 1;
  if (cpl <= 4) {
    if (a.n / 4 >= 6 * simds) r = 4;
    else if (a.n / 2 >= 6 * simds) r = 2;
  }
#define RZ_CASE(R_, C_) \
  if (r == R_ && cpl == C_) return launch_cfg<XT, UNIT, R_, C_>(a, stream);
  RZ_CASE(1, 1) RZ_CASE(1, 2) RZ_CASE(1, 4) RZ_CASE(1, 7) RZ_CASE(1, 8)
  RZ_CASE(2, 1) RZ_CASE(2, 2) RZ_CASE(2, 4)
  RZ_CASE(4, 1) RZ_CASE(4, 2) RZ_CASE(4, 4)
#undef RZ_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(const void* x, int x_dtype, const PackedView& w, void* y, int y_dtype,
                       void*, size_t, hipStream_t stream) {
  GemvArgs a;
  a.x = x;
  a.codes = w.codes;
  a.scales = w.scales;
  a.ts = w.tensor_scale;
  a.y = y;
  a.n = w.rows;
  a.k = w.cols;
  a.kind = w.kind;
  a.ydt = y_dtype;
  a.m0 = 6.0f + 0.5f * (float)w.off_half[0];
  a.m1 = 6.0f + 0.5f * (float)w.off_half[w.kind == kWeight ? 1 : 0];
  a.npass = 1;
  const bool unit2 = a.k % 32 == 0;
  a.nchunk = a.k / (unit2 ? 32 : 16);
  if (x_dtype == kF16) return unit2 ? dispatch<_Float16, 2>(a, stream) : dispatch<_Float16, 1>(a, stream);
  return unit2 ? dispatch<__bf16, 2>(a, stream) : dispatch<__bf16, 1>(a, stream);
}

}  // namespace rz
