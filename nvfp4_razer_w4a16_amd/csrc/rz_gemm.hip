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

// The same for the 128-element FP16-scale layout: the block's scale and
// special value come from its 16-bit word (metadata in bits 15-14).
template <typename XT>
__device__ __forceinline__ void decode_block_f16s(uint2 cw, uint32_t word, float m0, float m1, XT (&out)[16]) {
  const float sb = scale_of_f16word(word);
  const float sv = special_of_f16word(word, m0, m1) * sb;
#pragma unroll
  for (int j = 0; j < 16; j++) {
    const uint32_t nib = ((j < 8 ? cw.x : cw.y) >> (4 * (j & 7))) & 15u;
    const float mag = (float)fp4_mag_x2(nib & 7u) * (0.5f * sb);
    const float val = (nib == 8u) ? sv : ((nib & 8u) ? -mag : mag);
    out[j] = from_f32<XT>(val);
  }
}

constexpr int kBM = 128, kBN = 128, kBK = 32, kLds = kBK + 8;

// F16S: weights in the 128-element FP16-scale layout (one 16-bit scale word
// per 128 elements of a row) instead of 16-element blocks with byte scales.
template <typename XT, int KIND, typename OT, bool F16S = false>
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
        if constexpr (F16S) {
          const uint32_t word = ((const uint16_t*)scales)[gn * (k / 128) + kb / 8];
          decode_block_f16s<XT>(cw, word, m0, m1, vals);
        } else {
          const uint32_t sbyte = scales[gn * (k / 16) + kb];
          decode_block<KIND, XT>(cw, sbyte, m0, m1, vals);
        }
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
// For M >= 256 (prefill).  Eight waves, two per SIMD, laid out 2 (M) x 4 (N),
// each owning a 128 x 64 sub-tile (4 x 2 MFMA 32x32x16 tiles, 128 fp32
// accumulators per lane), so that while one wave of a SIMD waits on LDS or
// runs its decode the other keeps the matrix unit busy (four waves with
// 128 x 128 sub-tiles ran 20-28 % slower: one wave per SIMD left the matrix
// unit idle through its own decode and LDS waits).  Per K step each thread
// prefetches 64 bytes of x and half a weight row (32 elements) into registers
// while the waves run the step's MFMAs; then it writes the x bytes and the 32
// decoded values into the other LDS buffer.  The x tile's LDS rows are padded
// by 16 bytes so the 16-byte fragment reads of 32 consecutive rows hit
// distinct banks; the decoded weight tile is swizzled instead (see bpos).
//
// Decode (per pair of codes): the packed FP4 conversion, an exact multiply by
// sb, and a bit select that puts the block's SV * sb where the remapped code
// (converted to -0) sits; see decode_pair_impl.
constexpr int kTM = 256, kTN = 256, kTK = 64, kTS = kTK + 8;
// The decoded B tile has unpadded 128-byte rows whose 16-byte chunks are
// XOR-swizzled by row: chunk c of row r sits at position c ^ key(r) with
// key(r) = (r & 6) | ((r0 ^ r2 ^ r3) & 1) (r_i the bits of r).  A decode write
// instruction puts rows 4j..4j+3 (8 lanes) or 8j..8j+7 (16 lanes) and two
// chunks c, c + 4 of each row; a fragment read puts 8 or 16 consecutive rows
// at one chunk.  With this key every group of 8 lanes hits distinct 16-byte
// slots of a 128-byte bank window, and every group of 16 lanes distinct slots
// of a 256-byte window (row parity picking the half), so both accesses are
// conflict-free whether the LDS serves 128 or 256 bytes per cycle.  (The
// earlier key (r >> 1) & 7 was conflict-free only for the 256-byte case; this
// one is 4-6 % faster on the prefill shape, same outputs.)
constexpr int kBS = kTK;
__device__ __forceinline__ int bkey(int row) { return (row & 6) | ((row ^ (row >> 2) ^ (row >> 3)) & 1); }
__device__ __forceinline__ int bpos(int row, int chunk) { return row * kBS + ((chunk ^ bkey(row)) << 3); }

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

// The remapped code converts to -0, the int16 minimum of a packed pair; it is
// detected on the unscaled pair, so no rounding step can lose that sign.
__device__ __forceinline__ uint32_t remapped_mask(uint32_t p) {
  const short2_t q = __builtin_elementwise_max(__builtin_bit_cast(short2_t, p),
                                               (short2_t){(short)0x8001, (short)0x8001});
  const ushort2_t one = __builtin_bit_cast(ushort2_t, __builtin_bit_cast(uint32_t, q) ^ p);
  return __builtin_bit_cast(uint32_t, (ushort2_t){0, 0} - one);
}

// Replace the -0 halves of p by sv (both halves of svd hold sv ^ 0x8000, i.e.
// sv - 0x8000 mod 2^16): d = max_i16(p, 0x8001) ^ p is 1 exactly at -0, and p + d * svd puts
// 0x8000 + sv - 0x8000 = sv there (v_pk_max_i16, v_xor, v_pk_mad_u16).
__device__ __forceinline__ uint32_t insert_special(uint32_t p, uint32_t svd) {
  const short2_t q = __builtin_elementwise_max(__builtin_bit_cast(short2_t, p),
                                               (short2_t){(short)0x8001, (short)0x8001});
  const ushort2_t d = __builtin_bit_cast(ushort2_t, __builtin_bit_cast(uint32_t, q) ^ p);
  return __builtin_bit_cast(uint32_t, d * __builtin_bit_cast(ushort2_t, svd) +
                                          __builtin_bit_cast(ushort2_t, p));
}

// One dword (8 codes, all in one block) -> 4 packed 16-bit pairs, each stage
// applied to the four pairs before the next so independent work can fill the
// conversion and packed-integer latencies.
template <typename XT>
__device__ __forceinline__ uint4 decode_dword(uint32_t w, float sb, uint32_t svd) {
  uint32_t p[4];
  if constexpr (__is_same(XT, _Float16)) {
    half2_t h[4];
    h[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    h[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    h[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    h[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
    uint32_t mask[4];
#pragma unroll
    for (int i = 0; i < 4; i++) mask[i] = remapped_mask(__builtin_bit_cast(uint32_t, h[i]));
    const _Float16 s16 = (_Float16)sb;
#pragma unroll
    for (int i = 0; i < 4; i++) p[i] = __builtin_bit_cast(uint32_t, h[i] * (half2_t){s16, s16});
    // mask is taken before scaling; the scaled -0 may lose its sign
    const uint32_t svb2 = svd ^ 0x80008000u;  // back to SV*sb bits in both halves
#pragma unroll
    for (int i = 0; i < 4; i++) p[i] = (mask[i] & svb2) | (~mask[i] & p[i]);
  } else {
    float2_t f[4];
    f[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    f[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    f[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    f[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
#pragma unroll
    for (int i = 0; i < 4; i++)
      p[i] = insert_special(pack2<XT>(__builtin_fmaf(f[i][0], sb, -0.0f), __builtin_fmaf(f[i][1], sb, -0.0f)), svd);
  }
  return make_uint4(p[0], p[1], p[2], p[3]);
}

// One pair (byte `sel` of w) of the decode above; `sel` folds to a constant
// once the caller's loop is unrolled.
template <typename XT>
__device__ __forceinline__ uint32_t decode_one_pair(uint32_t w, int sel, float sb, uint32_t svd) {
  if constexpr (__is_same(XT, _Float16)) {
    half2_t h;
    switch (sel) {
      case 0: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0); break;
      case 1: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1); break;
      case 2: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2); break;
      default: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3); break;
    }
    const uint32_t mask = remapped_mask(__builtin_bit_cast(uint32_t, h));
    const _Float16 s16 = (_Float16)sb;
    const uint32_t v = __builtin_bit_cast(uint32_t, h * (half2_t){s16, s16});
    return (mask & (svd ^ 0x80008000u)) | (~mask & v);
  } else {
    float2_t f;
    switch (sel) {
      case 0: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
      case 1: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
      case 2: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
      default: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
    }
    return insert_special(pack2<XT>(__builtin_fmaf(f[0], sb, -0.0f), __builtin_fmaf(f[1], sb, -0.0f)), svd);
  }
}

// F16S: weights in the 128-element FP16-scale layout; a K step of 64 lies in
// one 128-element block, so one scale word per weight row and step gives both
// coefficients (computed from the word instead of the table).
//
// Workgroups 0 .. full-1 compute tiles 0 .. full-1 over all of K.  Any further
// workgroup j = blockIdx.x - full takes K half j % 2 of tile full + j / 2 and
// writes its (scaled) fp32 sums, unconverted, to the 256x256 slot j of part;
// tail_fold_kernel adds the two halves of each such tile into y.
template <typename XT, int KIND, typename OT, bool F16S = false>
__global__ __launch_bounds__(512) void gemm_tile256_kernel(const XT* __restrict__ x, int64_t m,
                                                      const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ ts,
                                                      const float* __restrict__ ts2, int64_t n,
                                                      int64_t k, float m0, float m1, OT* __restrict__ y,
                                                      int64_t full, float* __restrict__ part) {
  typedef typename Mfma32<XT>::V V;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  XT* As = (XT*)smem;
  XT* Bs = As + 2 * kTM * kTS;
  float2* lut = (float2*)(Bs + 2 * kTN * kBS);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t ntn = (n + kTN - 1) / kTN;
  int64_t tile = blockIdx.x;
  int kt0 = 0, ktiles = (int)(k / kTK), slot = -1;
  if (tile >= full) {  // one K half of a tail tile
    const int64_t j = tile - full;
    const int h0 = ktiles / 2;
    tile = full + j / 2;
    slot = (int)j;
    kt0 = (j & 1) ? h0 : 0;
    ktiles = (j & 1) ? ktiles - h0 : h0;
  }
  const int64_t m_base = (tile / ntn) * kTM;
  const int64_t n_base = (tile % ntn) * kTN;
  if (tid < 256) {
    const uint32_t b = (uint32_t)tid;
    const float sb = scale_of_byte<KIND>(b);
    const uint32_t svd = bits16<XT>(special_of_byte<KIND>(b, m0, m1) * sb) ^ 0x8000u;
    lut[b] = make_float2(sb, __builtin_bit_cast(float, svd | (svd << 16)));
  }
  // Two register sets: the tile two K steps ahead is in flight while the
  // next tile is decoded into LDS under the current tile's MFMAs.  Per K step
  // a thread carries 64 bytes of x and half a weight row (16 code bytes, 32
  // elements) with its row's four scale bytes.
  struct Stage {
    uint4 a[4];
    uint4 c;
    uint32_t s;
  };
  Stage st0, st1;
  // Raw buffer loads (descriptors cover this workgroup's rows only): rows past
  // m or n read zero without a branch, so the wait counters stay exact.
  typedef __amdgpu_buffer_rsrc_t Rsrc;
  constexpr int kOob = 0x40000000;
  const int rows_m = (int)min((int64_t)kTM, m - m_base), rows_n = (int)min((int64_t)kTN, n - n_base);
  const Rsrc xr = __builtin_amdgcn_make_buffer_rsrc((void*)(x + m_base * k), (short)0,
                                                    (int)(rows_m * k * (int64_t)sizeof(XT)), 0x00020000);
  const Rsrc cr = __builtin_amdgcn_make_buffer_rsrc((void*)(codes + n_base * (k / 2)), (short)0,
                                                    (int)(rows_n * (k / 2)), 0x00020000);
  const int64_t srb = F16S ? k / 64 : k / 16;  // scale bytes per weight row
  const Rsrc sr = __builtin_amdgcn_make_buffer_rsrc((void*)(scales + n_base * srb), (short)0,
                                                    (int)(rows_n * srb), 0x00020000);
  int xo[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int idx = i * 512 + tid;
    xo[i] = (idx >> 3) < rows_m ? (int)(((int64_t)(idx >> 3) * k + (idx & 7) * 8) * (int64_t)sizeof(XT)) : kOob;
  }
  const int br = tid >> 1, bh = tid & 1;  // the weight row and half this thread decodes
  const int co = br < rows_n ? (int)((int64_t)br * (k / 2)) + 16 * bh : kOob;
  const int so = br < rows_n ? (int)((int64_t)br * srb) : kOob;
  auto gload = [&](int kt, Stage& r) {
    const int k0 = (kt0 + kt) * kTK;
    if constexpr (F16S)
      r.s = __builtin_amdgcn_raw_buffer_load_b16(sr, so, (k0 / 128) * 2, 0);
    else
      r.s = __builtin_amdgcn_raw_buffer_load_b32(sr, so, k0 / 16, 0);
    const u32x4_t c0 = __builtin_amdgcn_raw_buffer_load_b128(cr, co, k0 / 2, 0);
    r.c = make_uint4(c0[0], c0[1], c0[2], c0[3]);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xr, xo[i], k0 * (int)sizeof(XT), 0);
      r.a[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  };
  auto cword = [](const uint4& c, int kk) { return kk == 0 ? c.x : kk == 1 ? c.y : kk == 2 ? c.z : c.w; };
  // (sb, SV * sb bits ^ 0x8000 in both halves) of 16-element block j (0..3) of a step
  auto coef = [&](uint32_t s, int j) -> float2 {
    if constexpr (F16S) {
      const float sb = scale_of_f16word(s);
      const uint32_t svd = bits16<XT>(special_of_f16word(s, m0, m1) * sb) ^ 0x8000u;
      return make_float2(sb, __builtin_bit_cast(float, svd | (svd << 16)));
    } else {
      return lut[(s >> (8 * j)) & 0xFFu];
    }
  };
  auto lstore = [&](const Stage& r, int buf) {
    XT* a = As + buf * kTM * kTS;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int idx = i * 512 + tid;
      *(uint4*)(a + (idx >> 3) * kTS + (idx & 7) * 8) = r.a[i];
    }
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const float2 f = coef(r.s, 2 * bh + (kk >> 1));
      *(uint4*)(Bs + buf * kTN * kBS + bpos(br, 4 * bh + kk)) =
          decode_dword<XT>(cword(r.c, kk), f.x, __builtin_bit_cast(uint32_t, f.y));
    }
  };
  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;

  auto step = [&](int kt, Stage& cur_stage, Stage& next_stage) {
    const int cur = kt & 1;
    gload(kt + 2 < ktiles ? kt + 2 : ktiles - 1, next_stage);
    float2 f[2];
#pragma unroll
    for (int j = 0; j < 2; j++) f[j] = coef(cur_stage.s, 2 * bh + j);
    const XT* a = As + cur * kTM * kTS;
    const XT* b = Bs + cur * kTN * kBS;
    V av[2][4], bv[2][2];
    auto frags = [&](int kk, V* ar, V* bq) {
#pragma unroll
      for (int i = 0; i < 4; i++)
        ar[i] = *(const V*)(a + (wm * 128 + i * 32 + (lane & 31)) * kTS + 16 * kk + 8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 2; j++)
        bq[j] = *(const V*)(b + bpos(wn * 64 + j * 32 + (lane & 31), 2 * kk + (lane >> 5)));
    };
    frags(0, av[0], bv[0]);
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      if (kk < 3) frags(kk + 1, av[(kk + 1) & 1], bv[(kk + 1) & 1]);
      XT* an = As + (cur ^ 1) * kTM * kTS;
      {
        const int idx = kk * 512 + tid;
        *(uint4*)(an + (idx >> 3) * kTS + (idx & 7) * 8) = cur_stage.a[kk];
      }
      const uint32_t w = cword(cur_stage.c, kk);
      const float2 fk = f[kk >> 1];
      const uint32_t svd = __builtin_bit_cast(uint32_t, fk.y);
      uint32_t dec[4];
#pragma unroll
      for (int g = 0; g < 4; g++) dec[g] = decode_one_pair<XT>(w, g, fk.x, svd);
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = Mfma32<XT>::run(av[kk & 1][i], bv[kk & 1][j], acc[i][j]);
      // one MFMA, then up to four VALU instructions of the pair decodes
#pragma unroll
      for (int g = 0; g < 8; g++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      *(uint4*)(Bs + (cur ^ 1) * kTN * kBS + bpos(br, 4 * bh + kk)) = make_uint4(dec[0], dec[1], dec[2], dec[3]);
    }
    __syncthreads();
  };

  gload(0, st0);
  gload(ktiles > 1 ? 1 : 0, st1);
  __syncthreads();
  lstore(st0, 0);
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < ktiles; kt += 2) {
    step(kt, st1, st0);
    step(kt + 1, st0, st1);
  }
  if (kt < ktiles) step(kt, st1, st0);
  // ts2: a second factor applied after the weight's tensor scale (the
  // activations' tensor scale of the W4A4 product), 1 when absent
  const float scale = *ts, scale2 = ts2 ? *ts2 : 1.0f;
  if (slot >= 0) {  // a K half: the whole 256x256 slot, rows and columns past m, n included
    float* p = part + (int64_t)slot * (kTM * kTN);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int lc = wn * 64 + j * 32 + (lane & 31);
#pragma unroll
        for (int e = 0; e < 16; e++) {
          const int lr = wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          p[lr * kTN + lc] = (acc[i][j][e] * scale) * scale2;
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int64_t gc = n_base + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int64_t gr = m_base + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (gr < m && gc < n) y[gr * n + gc] = from_f32<OT>((acc[i][j][e] * scale) * scale2);
      }
    }
}

// y of the tail tiles: the sum of the two K halves' slots.  blockIdx.y = tail
// tile t (tile full + t), blockIdx.x = 1024-element run of it; a thread adds
// four consecutive columns of one row.
template <typename OT>
__global__ __launch_bounds__(256) void tail_fold_kernel(const float* __restrict__ part, int64_t full,
                                                     int64_t m, int64_t n, OT* __restrict__ y) {
  const int64_t t = blockIdx.y, tile = full + t, ntn = (n + kTN - 1) / kTN;
  const int64_t m_base = (tile / ntn) * kTM, n_base = (tile % ntn) * kTN;
  const int idx = (blockIdx.x * 256 + threadIdx.x) * 4;
  const uint4 a = load_nt16(part + (2 * t) * (kTM * kTN) + idx);  // read once
  const uint4 b = load_nt16(part + (2 * t + 1) * (kTM * kTN) + idx);
  const int64_t gr = m_base + idx / kTN, gc = n_base + idx % kTN;
  if (gr >= m) return;
  const float v[4] = {__uint_as_float(a.x) + __uint_as_float(b.x), __uint_as_float(a.y) + __uint_as_float(b.y),
                      __uint_as_float(a.z) + __uint_as_float(b.z), __uint_as_float(a.w) + __uint_as_float(b.w)};
  OT* yp = y + gr * n + gc;
  if (gc + 4 <= n && ((uintptr_t)yp & (4 * sizeof(OT) - 1)) == 0) {  // one aligned vector store
    struct alignas(4 * sizeof(OT)) Q { OT e[4]; } q;
#pragma unroll
    for (int e = 0; e < 4; e++) q.e[e] = from_f32<OT>(v[e]);
    *(Q*)yp = q;
  } else {
#pragma unroll
    for (int e = 0; e < 4; e++)
      if (gc + e < n) yp[e] = from_f32<OT>(v[e]);
  }
}

// ---- small M (2..32): weight-streaming MFMA with split K -------------------------
//
// HBM-bound.  A wave owns 64 weight rows (4 groups of 16) for a K range; a
// workgroup's 4 waves split that range 4 ways and fold their partial tiles in
// LDS; a global split of K across workgroups (chosen so >= ~2k waves run)
// writes fp32 partials that skinny_reduce_kernel sums, scales by st and
// converts.  MFMA 16x16x32 (A = x rows, B = decoded weights): lane (c, q) =
// (l % 16, l / 16) loads 16 code bytes of weight row c covering 32
// consecutive k, k0 + 32q .. k0 + 32q + 31, and MFMA j (j = 0..3) of the
// 128-k window uses dword j of it, i.e. k0 + 32q + 8j .. +7, with the x
// fragment taken from the same k range (the MFMA sums over k, so any k order
// shared by A and B is valid).  Each dword lies in one 16-element block, so
// one scale byte serves it.
typedef __bf16 bf16x8s_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8s_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <typename XT> struct Mfma16;
template <> struct Mfma16<__bf16> {
  typedef bf16x8s_t V;
  static __device__ __forceinline__ floatx4 run(V a, V b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma16<_Float16> {
  typedef f16x8s_t V;
  static __device__ __forceinline__ floatx4 run(V a, V b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int kSkGroups = 4;      // 16-row weight groups per wave
constexpr int kSkRows = 16 * kSkGroups;

struct SkinnyPlan {
  int64_t wg_cols;   // workgroups along N (64 rows each)
  int split;         // global K split
  int64_t win_per_wave;  // 128-k windows per wave
};

static SkinnyPlan skinny_plan(int64_t n, int64_t k) {
  SkinnyPlan p;
  p.wg_cols = (n + kSkRows - 1) / kSkRows;
  const int64_t windows = (k + 127) / 128;
  const int64_t target_wgs = 4LL * device_cu_count();  // ~16 waves per CU
  int split = 1;
  // double the split while the grid is still small and every wave keeps >= 2
  // windows to pipeline
  while (split < 64 && p.wg_cols * split * 2 <= target_wgs && windows >= 4LL * split * 4) split *= 2;
  p.split = split;
  p.win_per_wave = (windows + 4LL * split - 1) / (4LL * split);
  return p;
}

template <typename XT, int KIND, int MT>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const XT* __restrict__ x, int m,
                                                          const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales,
                                                          int64_t n, int64_t k, float m0, float m1,
                                                          int64_t win_per_wave,
                                                          float* __restrict__ partial) {
  typedef typename Mfma16<XT>::V V;
  __shared__ floatx4 red[3][kSkGroups * MT][64];
  __shared__ float2 lut[256];  // scale byte -> (sb, SV * sb bits ^ 0x8000 in both halves)
  {
    const uint32_t b = threadIdx.x;
    const float sb = scale_of_byte<KIND>(b);
    const uint32_t svd = bits16<XT>(special_of_byte<KIND>(b, m0, m1) * sb) ^ 0x8000u;
    lut[b] = make_float2(sb, __builtin_bit_cast(float, svd | (svd << 16)));
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int64_t wg_cols = (n + kSkRows - 1) / kSkRows;
  const int64_t col_wg = blockIdx.x % wg_cols;
  const int split_id = (int)(blockIdx.x / wg_cols);
  const int64_t nwin = (k + 127) / 128;
  const int64_t w_begin = ((int64_t)split_id * 4 + wave) * win_per_wave;
  const int64_t w_end = w_begin + win_per_wave < nwin ? w_begin + win_per_wave : nwin;
  const int64_t row_base = col_wg * kSkRows;

  floatx4 acc[kSkGroups][MT];
#pragma unroll
  for (int g = 0; g < kSkGroups; g++)
#pragma unroll
    for (int t = 0; t < MT; t++) acc[g][t] = (floatx4){0.f, 0.f, 0.f, 0.f};

  struct Win {
    uint4 cw[kSkGroups];
    uint32_t sw[kSkGroups];
    V xa[MT][4];
  };
  auto load_win = [&](int64_t w, Win& r) {
    const int64_t kq = w * 128 + 32 * q;  // this lane's 32-k slice
    const bool kvalid = kq < k;
#pragma unroll
    for (int g = 0; g < kSkGroups; g++) {
      const int64_t row = row_base + 16 * g + c;
      if (row < n && kvalid) {
        r.cw[g] = load_nt16(codes + row * (k / 2) + kq / 2);
        r.sw[g] = *(const uint16_t*)(scales + row * (k / 16) + kq / 16);
      } else {
        r.cw[g] = make_uint4(0, 0, 0, 0);
        r.sw[g] = 0;
      }
    }
#pragma unroll
    for (int t = 0; t < MT; t++) {
      const int row = 16 * t + c;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < m && kvalid) v = *(const uint4*)(x + (int64_t)row * k + kq + 8 * j);
        r.xa[t][j] = __builtin_bit_cast(V, v);
      }
    }
  };
  auto compute_win = [&](const Win& r) {
#pragma unroll
    for (int g = 0; g < kSkGroups; g++) {
      const float2 f0 = lut[r.sw[g] & 0xFFu], f1 = lut[(r.sw[g] >> 8) & 0xFFu];
      const uint32_t d[4] = {r.cw[g].x, r.cw[g].y, r.cw[g].z, r.cw[g].w};
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float2 f = j < 2 ? f0 : f1;
        const uint4 bv = decode_dword<XT>(d[j], f.x, __builtin_bit_cast(uint32_t, f.y));
        const V b = __builtin_bit_cast(V, bv);
#pragma unroll
        for (int t = 0; t < MT; t++) acc[g][t] = Mfma16<XT>::run(r.xa[t][j], b, acc[g][t]);
      }
    }
  };
  // two register sets, loads for the next window in flight during each decode
  Win r0, r1;
  if (w_begin < w_end) load_win(w_begin, r0);
  for (int64_t w = w_begin; w < w_end; w += 2) {
    if (w + 1 < w_end) load_win(w + 1, r1);
    compute_win(r0);
    if (w + 2 < w_end) load_win(w + 2, r0);
    if (w + 1 < w_end) compute_win(r1);
  }

  // fold the 4 waves' K slices
  if (wave > 0) {
#pragma unroll
    for (int g = 0; g < kSkGroups; g++)
#pragma unroll
      for (int t = 0; t < MT; t++) red[wave - 1][g * MT + t][lane] = acc[g][t];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int g = 0; g < kSkGroups; g++)
#pragma unroll
      for (int t = 0; t < MT; t++) {
        floatx4 v = acc[g][t];
#pragma unroll
        for (int o = 0; o < 3; o++) v += red[o][g * MT + t][lane];
        // C layout: lane (c, q) holds rows 4q .. 4q+3 of column c
        const int64_t col = row_base + 16 * g + c;
        if (col < n) {
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int row = 16 * t + 4 * q + i;
            if (row < m) partial[((int64_t)split_id * m + row) * n + col] = v[i];
          }
        }
      }
  }
}

// ---- batches of 5..32 rows: weight-streaming MFMA, x unit shared in LDS ---------
//
// HBM-bound like the small-batch kernel, but x is dense: for every 256-element
// K unit the workgroup stages x[M, 256] once in LDS (row stride 528 bytes, so
// the 16-byte fragment reads of 16 rows hit distinct banks) and its four
// waves each stream TW 16-row weight tiles through a padded per-wave stage
// (coalesced 16-byte loads covering whole 128-byte row segments).  Lane
// (q, c) decodes 64 elements of weight row c -- value * sb with the remapped
// code replaced by SV * sb (decode_dword) -- into the B operands of 8
// v_mfma_f32_16x16x32 MFMAs (K slot 8q + t of MFMA i = element 64q + 8i + t
// of the unit), and reads the matching x fragments as A.  The next unit's
// loads are in flight during each unit; a global K split, when the rows are
// too few to fill the GPU, goes through fp32 partials and skinny_reduce_kernel.
constexpr int kBxRow = 256 + 8;                    // staged x halves per row
constexpr int kBStage = 16 * 144 + 16 * 16;        // one 16-row tile unit: codes + scales

// F16S: weights in the 128-element FP16-scale layout: a unit's scales are one
// dword (two words) per row, staged by lanes 0..15; a lane's 64 elements lie
// in one 128-element block, whose word gives both coefficients.
template <typename XT, int KIND, int MT, int TW, bool F16S = false>
__global__ __launch_bounds__(256) void gemm_batch_kernel(const XT* __restrict__ x, int m,
                                                         const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ ts, int64_t n,
                                                         int64_t k, float m0, float m1, int wg_rows,
                                                         int upw, float* __restrict__ partial,
                                                         void* __restrict__ y, int ydt) {
  typedef typename Mfma16<XT>::V V;
  typedef __amdgpu_buffer_rsrc_t Rsrc;
  constexpr int kOob = 0x40000000;
  __shared__ float2 lut[256];  // scale byte -> (sb, SV * sb bits ^ 0x8000 in both halves)
  __shared__ __attribute__((aligned(16))) XT xs[2][MT * 16][kBxRow];
  __shared__ __attribute__((aligned(16))) uint8_t stage[4][2][TW][kBStage];
  {
    const uint32_t b = threadIdx.x;
    const float sb = scale_of_byte<KIND>(b);
    const uint32_t svd = bits16<XT>(special_of_byte<KIND>(b, m0, m1) * sb) ^ 0x8000u;
    lut[b] = make_float2(sb, __builtin_bit_cast(float, svd | (svd << 16)));
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, q = lane >> 4;
  const int sid = blockIdx.x / wg_rows;                       // K split index
  const int64_t row0 = (int64_t)(blockIdx.x % wg_rows) * (64 * TW) + wave * (16 * TW);
  const int nunits = (int)(k / 256);
  const int u0 = sid * upw, u1 = min(nunits, u0 + upw);
  const int rcb = (int)(k / 2), rsb = (int)(F16S ? k / 64 : k / 16);
  const int rows_w = (int)max((int64_t)0, min((int64_t)(16 * TW), n - row0));
  const Rsrc crs = __builtin_amdgcn_make_buffer_rsrc((void*)(codes + (row0 < n ? row0 : 0) * rcb), (short)0,
                                                     rows_w * rcb, 0x00020000);
  const Rsrc srs = __builtin_amdgcn_make_buffer_rsrc((void*)(scales + (row0 < n ? row0 : 0) * rsb), (short)0,
                                                     rows_w * rsb, 0x00020000);
  const Rsrc xrs = __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)((int64_t)m * k * 2), 0x00020000);

  // per-unit loads: x chunks (MT * 16 rows x 32 chunks of 16 bytes, 2 * MT per
  // thread), this wave's codes (lane i: row i >> 3 (+8), bytes 16 * (i & 7))
  // and scales (lane i: row i >> 2, bytes 4 * (i & 3)) for each of its tiles
  struct Regs {
    u32x4_t xv[2 * MT];
    u32x4_t c0[TW], c1[TW];
    uint32_t s[TW];
  };
  int xvo[2 * MT];
#pragma unroll
  for (int j = 0; j < 2 * MT; j++) {
    const int ch = tid + 256 * j, r = ch >> 5, cc = ch & 31;
    xvo[j] = r < m ? (int)(((int64_t)r * k + cc * 8) * 2) : kOob;
  }
  const int lr = lane >> 3, lb = (lane & 7) * 16;
  int cvo0[TW], cvo1[TW], svo[TW];
#pragma unroll
  for (int t = 0; t < TW; t++) {
    cvo0[t] = 16 * t + lr < rows_w ? (16 * t + lr) * rcb + lb : kOob;
    cvo1[t] = 16 * t + lr + 8 < rows_w ? (16 * t + lr + 8) * rcb + lb : kOob;
    if (F16S)
      svo[t] = lane < 16 && 16 * t + lane < rows_w ? (16 * t + lane) * rsb : kOob;
    else
      svo[t] = 16 * t + (lane >> 2) < rows_w ? (16 * t + (lane >> 2)) * rsb + (lane & 3) * 4 : kOob;
  }
  auto load_unit = [&](Regs& r, int u) {
    const bool ok = u < u1;
    const int xso = ok ? u * 512 : kOob, cso = ok ? u * 128 : kOob, sso = ok ? u * (F16S ? 4 : 16) : kOob;
#pragma unroll
    for (int j = 0; j < 2 * MT; j++) r.xv[j] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xvo[j], xso, 0);
#pragma unroll
    for (int t = 0; t < TW; t++) {
      r.c0[t] = __builtin_amdgcn_raw_buffer_load_b128(crs, cvo0[t], cso, 2);
      r.c1[t] = __builtin_amdgcn_raw_buffer_load_b128(crs, cvo1[t], cso, 2);
      r.s[t] = __builtin_amdgcn_raw_buffer_load_b32(srs, svo[t], sso, 0);
    }
  };
  auto store_unit = [&](const Regs& r, int buf) {
#pragma unroll
    for (int j = 0; j < 2 * MT; j++) {
      const int ch = tid + 256 * j;
      *(u32x4_t*)(&xs[buf][ch >> 5][(ch & 31) * 8]) = r.xv[j];
    }
#pragma unroll
    for (int t = 0; t < TW; t++) {
      uint8_t* st = stage[wave][buf][t];
      *(u32x4_t*)(st + lr * 144 + lb) = r.c0[t];
      *(u32x4_t*)(st + (lr + 8) * 144 + lb) = r.c1[t];
      if (!F16S)
        *(uint32_t*)(st + 16 * 144 + lane * 4) = r.s[t];
      else if (lane < 16)
        *(uint32_t*)(st + 16 * 144 + lane * 16) = r.s[t];
    }
  };

  floatx4 acc[TW][MT];
#pragma unroll
  for (int t = 0; t < TW; t++)
#pragma unroll
    for (int mt = 0; mt < MT; mt++) acc[t][mt] = (floatx4){0.f, 0.f, 0.f, 0.f};

  auto compute_unit = [&](int buf) {
#pragma unroll
    for (int t = 0; t < TW; t++) {
      const uint8_t* st = stage[wave][buf][t];
      const u32x4_t lo = *(const u32x4_t*)(st + c * 144 + 32 * q);
      const u32x4_t hi = *(const u32x4_t*)(st + c * 144 + 32 * q + 16);
      const uint32_t sw = F16S ? *(const uint32_t*)(st + 16 * 144 + c * 16)
                               : *(const uint32_t*)(st + 16 * 144 + c * 16 + 4 * q);
      const uint32_t cw[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      float2 f[4];
      if constexpr (F16S) {
        const uint32_t wd = (sw >> (16 * (q >> 1))) & 0xFFFFu;  // block (64 q) / 128 of the unit
        const float sb = scale_of_f16word(wd);
        const uint32_t svd = bits16<XT>(special_of_f16word(wd, m0, m1) * sb) ^ 0x8000u;
        f[0] = make_float2(sb, __builtin_bit_cast(float, svd | (svd << 16)));
#pragma unroll
        for (int b = 1; b < 4; b++) f[b] = f[0];
      } else {
#pragma unroll
        for (int b = 0; b < 4; b++) f[b] = lut[(sw >> (8 * b)) & 0xFFu];
      }
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint4 bv = decode_dword<XT>(cw[i], f[i >> 1].x, __builtin_bit_cast(uint32_t, f[i >> 1].y));
        const V bb = __builtin_bit_cast(V, bv);
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
          const V xa = *(const V*)(&xs[buf][mt * 16 + c][64 * q + 8 * i]);
          acc[t][mt] = Mfma16<XT>::run(xa, bb, acc[t][mt]);
        }
      }
    }
  };

  Regs rg;
  load_unit(rg, u0);
  __syncthreads();  // lut
  store_unit(rg, 0);
  load_unit(rg, u0 + 1);
  __syncthreads();
  for (int u = u0; u < u1; u++) {
    const int buf = (u - u0) & 1;
    compute_unit(buf);
    store_unit(rg, buf ^ 1);
    load_unit(rg, u + 2);
    __syncthreads();
  }

  // D layout: lane (q, c) holds rows 4q .. 4q+3 (x rows mt * 16 + ...) of column
  // c (weight row row0 + 16 t + c)
  const float st = *ts;
#pragma unroll
  for (int t = 0; t < TW; t++) {
    const int64_t col = row0 + 16 * t + c;
    if (col >= n) continue;
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int xr = mt * 16 + 4 * q + e;
        if (xr >= m) continue;
        const float v = acc[t][mt][e];
        if (partial) {
          partial[((int64_t)sid * m + xr) * n + col] = v;
        } else {
          const int64_t o = (int64_t)xr * n + col;
          if (ydt == kF32) ((float*)y)[o] = v * st;
          else if (ydt == kF16) ((_Float16*)y)[o] = (_Float16)(v * st);
          else ((__bf16*)y)[o] = (__bf16)(v * st);
        }
      }
  }
}

struct BatchPlan {
  int tw, split, upw;
  int64_t wg_rows;
};

// One 16-row tile per wave; a global K split while the grid stays under a
// row-count dependent target (more rows carry more MFMA and x work per weight
// byte, so need fewer workgroups to cover HBM latency) and every split keeps
// >= 2 units.
static BatchPlan batch_plan(int64_t m, int64_t n, int64_t k, bool untrimmed = false) {
  BatchPlan p;
  const int64_t tiles = (n + 15) / 16;
  const int64_t cus = device_cu_count();
  p.tw = 1;
  p.wg_rows = (tiles + 4 * p.tw - 1) / (4 * p.tw);
  const int64_t nunits = k / 256;
  const int64_t target = m <= 16 ? 8 * cus : 3 * cus / 2;
  p.split = 1;
  while (p.wg_rows * p.split * 2 <= target && nunits / (2 * p.split) >= 2) p.split *= 2;
  if (untrimmed)  // the most splits: one 256-element unit per workgroup, at most 32
    while (p.split < 32 && nunits / (2 * p.split) >= 1) p.split *= 2;
  p.upw = (int)((nunits + p.split - 1) / p.split);
  return p;
}

static bool use_batch(int64_t m, int64_t k) { return m >= 3 && m <= 32 && k >= 256 && k % 256 == 0 && k < (1LL << 24); }
// The FP16-scale layout has no small-batch kernel: the batch kernel from 2 rows.
static bool use_batch_f16s(int64_t m, int64_t k) { return m == 2 ? use_batch(3, k) : use_batch(m, k); }

template <typename OT>
__global__ __launch_bounds__(256) void skinny_reduce_kernel(const float* __restrict__ partial,
                                                            int split, int64_t mn,
                                                            const float* __restrict__ ts,
                                                            OT* __restrict__ y) {
  const float st = *ts;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < mn; i += (int64_t)gridDim.x * 256) {
    // the split partials are independent loads: issue eight at a time
    float v = 0.0f;
    int s = 0;
    for (; s + 8 <= split; s += 8) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; j++) p[j] = partial[(int64_t)(s + j) * mn + i];
#pragma unroll
      for (int j = 0; j < 8; j++) v += p[j];
    }
    if (s + 4 <= split) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; j++) p[j] = partial[(int64_t)(s + j) * mn + i];
#pragma unroll
      for (int j = 0; j < 4; j++) v += p[j];
      s += 4;
    }
    if (s + 2 <= split) {
      const float p0 = partial[(int64_t)s * mn + i], p1 = partial[(int64_t)(s + 1) * mn + i];
      v += p0;
      v += p1;
      s += 2;
    }
    if (s < split) v += partial[(int64_t)s * mn + i];
    y[i] = from_f32<OT>(v * st);
  }
}

// Routing on the default layout (no workspace for the first two): three to
// eight rows with K % 256 == 0 go to the block-diagonal streaming kernel,
// except three and four rows on weights under 128M elements; those and two
// rows go to the MFMA small-batch kernel where it covers the shape; the batch
// kernel takes up to 32 rows, the skinny split-K kernel the shapes none covers.
static bool use_bdiag(int64_t m, int64_t n, int64_t k) {
  if (m < 3 || m > 8 || !bdiag_supported(m, n, k)) return false;
  return m >= 5 || n * k >= (128LL << 20);
}

static bool use_smallm(int64_t m, int64_t n, int64_t k) {
  if (m < 2 || m > 4 || !smallm_supported(m, n, k)) return false;
  return m == 2 || n * k < (128LL << 20);
}

size_t gemm_ws_need(int64_t m, int64_t n, int64_t k, bool f16s, bool untrimmed) {
  if (f16s) {
    if (fp16s_supported(m, n, k) || !use_batch_f16s(m, k)) return 0;
    const BatchPlan p = batch_plan(m, n, k, untrimmed);
    return p.split > 1 ? (size_t)p.split * (size_t)m * (size_t)n * sizeof(float) : 0;
  }
  if (use_bdiag(m, n, k) || use_smallm(m, n, k)) return 0;
  if (use_batch(m, k)) {
    const BatchPlan p = batch_plan(m, n, k, untrimmed);
    return p.split > 1 ? (size_t)p.split * (size_t)m * (size_t)n * sizeof(float) : 0;
  }
  if (m < 2 || m > 32 || k % 32 != 0) return 0;
  const SkinnyPlan p = skinny_plan(n, k);
  return (size_t)p.split * (size_t)m * (size_t)n * sizeof(float);
}

// Enough for either layout (two rows need no workspace on the default layout
// but may on the FP16-scale one).
size_t gemm_ws_bytes(int64_t m, int64_t n, int64_t k) {
  const size_t a = gemm_ws_need(m, n, k, false), b = gemm_ws_need(m, n, k, true);
  const size_t c = prefill_ws_bytes(m, n, k);
  return a > b ? (a > c ? a : c) : (b > c ? b : c);
}

static bool tile256_fits(int64_t m, int64_t k, size_t xsize) {
  return m >= kTM && k % kTK == 0 && (int64_t)kTM * k * (int64_t)xsize < (1LL << 30);
}

// One 256x256 tile per CU at a time: a tile count just past a multiple of the
// CU count leaves a last round that runs on few CUs.  When that round would
// fill at most half of them, its tiles are split into two K halves (twice the
// workgroups, half the steps each), which costs two fp32 partial tiles per
// tail tile in the workspace and one fold launch.  Returns the tail tiles.
static int64_t tail_tiles(int64_t m, int64_t n, int64_t k) {
  const int64_t tiles = ((m + kTM - 1) / kTM) * ((n + kTN - 1) / kTN), cus = device_cu_count();
  const int64_t tail = tiles % cus;
  if (tiles <= cus || tail == 0 || 2 * tail > cus || k / kTK < 2) return 0;
  return tail;
}

size_t prefill_ws_bytes(int64_t m, int64_t n, int64_t k) {
  if (!tile256_fits(m, k, 2)) return 0;
  return (size_t)tail_tiles(m, n, k) * 2 * kTM * kTN * sizeof(float);
}

template <typename XT, int KIND, typename OT, bool F16S = false>
static hipError_t run_tile256(const XT* x, int64_t m, const PackedView& w, OT* y, const float* ts2,
                              void* ws, size_t wsb, hipStream_t stream) {
  const int64_t n = w.rows, k = w.cols;
  const float m0 = 6.0f + 0.5f * (float)w.off_half[0];
  const float m1 = 6.0f + 0.5f * (float)w.off_half[KIND == kWeight ? 1 : 0];
  auto kern = gemm_tile256_kernel<XT, KIND, OT, F16S>;
  const size_t lds = (size_t)2 * (kTM * kTS + kTN * kBS) * sizeof(XT) + 256 * sizeof(float2);
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((m + kTM - 1) / kTM) * ((n + kTN - 1) / kTN);
  // the tail split only with a workspace that holds its partial tiles
  int64_t tail = tail_tiles(m, n, k);
  if (!ws || ((uintptr_t)ws & 15) || wsb < (size_t)tail * 2 * kTM * kTN * sizeof(float)) tail = 0;
  const int64_t full = tiles - tail;
  hipLaunchKernelGGL(kern, dim3((unsigned)(full + 2 * tail)), dim3(512), lds, stream, x, m, w.codes, w.scales,
                     w.tensor_scale, ts2, n, k, m0, m1, y, full, (float*)ws);
  if (tail > 0)
    hipLaunchKernelGGL(tail_fold_kernel<OT>, dim3(kTM * kTN / 1024, (unsigned)tail), dim3(256), 0, stream,
                       (const float*)ws, full, m, n, y);
  return hipGetLastError();
}

// The batch kernel (3..32 rows; 2..32 rows on the FP16-scale layout), with
// the global K split's partial sums reduced by skinny_reduce_kernel.
template <typename XT, int KIND, typename OT, bool F16S>
static hipError_t run_batch(const XT* x, int64_t m, const PackedView& w, OT* y, void* ws, hipStream_t stream) {
  const int64_t n = w.rows, k = w.cols;
  const float m0 = 6.0f + 0.5f * (float)w.off_half[0];
  const float m1 = 6.0f + 0.5f * (float)w.off_half[KIND == kWeight ? 1 : 0];
  {
    const BatchPlan p = batch_plan(m, n, k, (w.flags & kFlagUntrimmed) != 0);
    float* partial = p.split > 1 ? (float*)ws : nullptr;
    if (p.split > 1 && !partial) return hipErrorInvalidValue;
    const int ydt = sizeof(OT) == 4 ? kF32 : __is_same(OT, _Float16) ? kF16 : kBF16;
    const int64_t grid = p.wg_rows * p.split;
#define RZ_BATCH(MT_, TW_)                                                                                \
  hipLaunchKernelGGL((gemm_batch_kernel<XT, KIND, MT_, TW_, F16S>), dim3((unsigned)grid), dim3(256), 0, stream, x, \
                     (int)m, w.codes, w.scales, w.tensor_scale, n, k, m0, m1, (int)p.wg_rows, p.upw,        \
                     partial, (void*)y, ydt)
    if (m <= 16) {
      if (p.tw == 2) RZ_BATCH(1, 2); else RZ_BATCH(1, 1);
    } else {
      if (p.tw == 2) RZ_BATCH(2, 2); else RZ_BATCH(2, 1);
    }
#undef RZ_BATCH
    if (p.split > 1) {
      const int64_t mn = m * n;
      int64_t g2 = (mn + 255) / 256;
      if (g2 > 4LL * device_cu_count()) g2 = 4LL * device_cu_count();
      hipLaunchKernelGGL((skinny_reduce_kernel<OT>), dim3((unsigned)g2), dim3(256), 0, stream, partial,
                         p.split, mn, w.tensor_scale, y);
    }
    return hipGetLastError();
  }
}

// The 128-element FP16-scale layout: the streaming kernel for 2..32 rows
// (K % 256 == 0; 17..32 on large weights), the batch kernel up to 32 rows
// otherwise, the prefill kernel where it
// fits, else the generic tile kernel.
template <typename XT, int KIND, typename OT>
static hipError_t run_gemm_f16s(const XT* x, int64_t m, const PackedView& w, OT* y, void* ws,
                                size_t wsb, hipStream_t stream) {
  const int64_t n = w.rows, k = w.cols;
  if (k % 128 != 0) return hipErrorInvalidValue;
  if (KIND == kWeight && fp16s_supported(m, n, k))
    return launch_bdiag(x, __is_same(XT, __bf16) ? kBF16 : kF16, m, w, y,
                        sizeof(OT) == 4 ? kF32 : __is_same(OT, _Float16) ? kF16 : kBF16, stream);
  if (use_batch_f16s(m, k)) return run_batch<XT, KIND, OT, true>(x, m, w, y, ws, stream);
  if (tile256_fits(m, k, sizeof(XT))) return run_tile256<XT, KIND, OT, true>(x, m, w, y, nullptr, ws, wsb, stream);
  const float m0 = 6.0f + 0.5f * (float)w.off_half[0];
  const float m1 = 6.0f + 0.5f * (float)w.off_half[KIND == kWeight ? 1 : 0];
  dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
  hipLaunchKernelGGL((gemm_kernel<XT, KIND, OT, true>), grid, dim3(256), 0, stream, x, m, w.codes,
                     w.scales, w.tensor_scale, n, k, m0, m1, y);
  return hipGetLastError();
}

template <typename XT, int KIND, typename OT>
static hipError_t run_gemm(const XT* x, int64_t m, const PackedView& w, OT* y, void* ws, size_t wsb,
                           hipStream_t stream) {
  if (!default_layout(w)) return run_gemm_f16s<XT, KIND, OT>(x, m, w, y, ws, wsb, stream);
  const int64_t n = w.rows, k = w.cols;
  const float m0 = 6.0f + 0.5f * (float)w.off_half[0];
  const float m1 = 6.0f + 0.5f * (float)w.off_half[KIND == kWeight ? 1 : 0];
  if (use_batch(m, k)) return run_batch<XT, KIND, OT, false>(x, m, w, y, ws, stream);
  if (m >= 2 && m <= 32 && k % 32 == 0 && ws != nullptr) {
    const SkinnyPlan p = skinny_plan(n, k);
    float* partial = (float*)ws;
    const int64_t grid = p.wg_cols * p.split;
    if (m <= 16)
      hipLaunchKernelGGL((gemm_skinny_kernel<XT, KIND, 1>), dim3((unsigned)grid), dim3(256), 0, stream,
                         x, (int)m, w.codes, w.scales, n, k, m0, m1, p.win_per_wave, partial);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<XT, KIND, 2>), dim3((unsigned)grid), dim3(256), 0, stream,
                         x, (int)m, w.codes, w.scales, n, k, m0, m1, p.win_per_wave, partial);
    const int64_t mn = m * n;
    int64_t g2 = (mn + 255) / 256;
    if (g2 > 4LL * device_cu_count()) g2 = 4LL * device_cu_count();
    hipLaunchKernelGGL((skinny_reduce_kernel<OT>), dim3((unsigned)g2), dim3(256), 0, stream, partial,
                       p.split, mn, w.tensor_scale, y);
    return hipGetLastError();
  }
  if (tile256_fits(m, k, sizeof(XT))) return run_tile256<XT, KIND, OT>(x, m, w, y, nullptr, ws, wsb, stream);
  dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
  hipLaunchKernelGGL((gemm_kernel<XT, KIND, OT>), grid, dim3(256), 0, stream, x, m, w.codes,
                     w.scales, w.tensor_scale, n, k, m0, m1, y);
  return hipGetLastError();
}

template <typename XT, int KIND>
static hipError_t gemm_out_dispatch(const XT* x, int64_t m, const PackedView& w, void* y,
                                    int y_dtype, void* ws, size_t wsb, hipStream_t stream) {
  if (y_dtype == kF32) return run_gemm<XT, KIND>(x, m, w, (float*)y, ws, wsb, stream);
  if (y_dtype == kF16) return run_gemm<XT, KIND>(x, m, w, (_Float16*)y, ws, wsb, stream);
  return run_gemm<XT, KIND>(x, m, w, (__bf16*)y, ws, wsb, stream);
}

template <typename XT, int KIND>
static hipError_t tile256_out_dispatch(const XT* x, int64_t m, const PackedView& w, void* y, int y_dtype,
                                       const float* ts2, void* ws, size_t wsb, hipStream_t stream) {
  if (y_dtype == kF32) return run_tile256<XT, KIND>(x, m, w, (float*)y, ts2, ws, wsb, stream);
  if (y_dtype == kF16) return run_tile256<XT, KIND>(x, m, w, (_Float16*)y, ts2, ws, wsb, stream);
  return run_tile256<XT, KIND>(x, m, w, (__bf16*)y, ts2, ws, wsb, stream);
}

bool gemm_prefill_fits(int64_t m, int64_t k, int x_dtype) { return tile256_fits(m, k, 2); }

hipError_t launch_gemm_prefill_scaled(const void* x, int x_dtype, int64_t m, const PackedView& w, void* y,
                                      int y_dtype, const float* ts2, void* ws, size_t wsb, hipStream_t stream) {
  if (!tile256_fits(m, w.cols, 2)) return hipErrorNotSupported;
  if (x_dtype == kF16) {
    if (w.kind == kWeight) return tile256_out_dispatch<_Float16, kWeight>((const _Float16*)x, m, w, y, y_dtype, ts2, ws, wsb, stream);
    return tile256_out_dispatch<_Float16, kAct>((const _Float16*)x, m, w, y, y_dtype, ts2, ws, wsb, stream);
  }
  if (w.kind == kWeight) return tile256_out_dispatch<__bf16, kWeight>((const __bf16*)x, m, w, y, y_dtype, ts2, ws, wsb, stream);
  return tile256_out_dispatch<__bf16, kAct>((const __bf16*)x, m, w, y, y_dtype, ts2, ws, wsb, stream);
}

hipError_t launch_gemm(const void* x, int x_dtype, int64_t m, const PackedView& w, void* y,
                       int y_dtype, void* ws, size_t wsb, hipStream_t stream) {
  if (default_layout(w) && use_bdiag(m, w.rows, w.cols)) return launch_bdiag(x, x_dtype, m, w, y, y_dtype, stream);
  if (default_layout(w) && use_smallm(m, w.rows, w.cols)) return launch_smallm(x, x_dtype, m, w, y, y_dtype, stream);
  if (!default_layout(w) && (w.blog2 != 7 || w.sfmt != 1)) return hipErrorNotSupported;
  if (x_dtype == kF16) {
    if (w.kind == kWeight) return gemm_out_dispatch<_Float16, kWeight>((const _Float16*)x, m, w, y, y_dtype, ws, wsb, stream);
    return gemm_out_dispatch<_Float16, kAct>((const _Float16*)x, m, w, y, y_dtype, ws, wsb, stream);
  }
  if (w.kind == kWeight) return gemm_out_dispatch<__bf16, kWeight>((const __bf16*)x, m, w, y, y_dtype, ws, wsb, stream);
  return gemm_out_dispatch<__bf16, kAct>((const __bf16*)x, m, w, y, y_dtype, ws, wsb, stream);
}

}  // namespace rz
