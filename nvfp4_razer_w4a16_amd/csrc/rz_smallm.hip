// rz_smallm.hip -- W4A16 product for 1..4 activation rows, y[M, N] = x[M, K] * W^T,
// with the dot products on gfx950 MFMA and the RaZeR weights decoded in
// registers.
//
// "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
// Remapping" (papernotes.org notes), Key design 3: weight-only GEMV/GEMM
// kernels decode the packed weights inside the kernel; "Technical Summary:
// RaZeR ..." (gist.science), §2.3 and §4 (decode and small batches).  The
// pages' kernel is prior art only.  This one is HBM-bound by design: the only
// per-element vector work is the packed FP4 conversion and one packed int16 max.
//
// v_mfma_f32_16x16x32_{f16,bf16}: D[16 x 16] += A[16 x 32] * B[32 x 16].  Lane
// l = c + 16 * q holds A row c, K slots 8q .. 8q+7; B column c, K slots
// 8q .. 8q+7; and D rows 4q .. 4q+3 of column c.
//   - B (weights): column c = weight row c of a 16-row tile; K slots 8q .. 8q+7
//     of MFMA i are elements 8i .. 8i+7 of lane q's slice of the K group, i.e.
//     byte pairs of code dword i, so B comes straight from the conversion.
//   - A (x, block-diagonal): row r = (vector mv, block slot s) with
//     r = mv * S + s; A[r][k] = x_mv[k] where K slot k belongs to block slot s,
//     else 0.  So D[r][c] is the dot of x_mv with ONE 16-element block of
//     weight row c, and the block scale can be applied per output element.
//     Each wave copies the x of its K groups to LDS once, one section per
//     group followed by 16 zero bytes; a lane whose slot lies in its K-slot
//     group reads its 8 x values from the section, every other lane reads the
//     zero bytes, so A costs one LDS read per MFMA and no vector work.
// A K group holds S = 16 / M blocks (256 / M elements, G = 8 / M MFMAs); lane
// q's slice is blocks q * S / 4 .. of it.  For every block two products are
// formed: d0 with the converted codes q and d1 with max(q, -0.25) as int16,
// which replaces only the remapped code (it converts to -0, the smallest
// int16 pattern) by -0.25; the block value is d0 + SV * S_x =
// d0 * (1 + 4 SV) - 4 SV * d1 with S_x the sum of x over remapped positions.
// A 256-entry LDS table holds both coefficients times the block scale.  The
// scale bytes a lane needs (weight row c, the four slots of its D rows) are
// one aligned dword of the scale row.
//
// Work split: a workgroup of KS waves owns one 16-row tile; wave w covers a
// contiguous range of 256-element K units with the loads of the next two units
// in flight while one is multiplied; the KS partial sums meet in LDS.
#include "rz_device.h"
#include "rz_launch.h"

namespace rz {

namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short short2_t __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

constexpr int kRsrcWord3 = 0x00020000;  // gfx950 raw buffer, 32-bit data format
constexpr int kOob = 0x40000000;        // past any num_records, also when added twice
constexpr int kNt = 2;                  // non-temporal: weights are read once

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, kRsrcWord3);
}

template <typename XT> struct Ops;
template <> struct Ops<_Float16> {
  typedef f16x8_t V;
  static constexpr uint32_t kQuarterNeg2 = 0xB400B400u;  // -0.25 in both fp16 halves
  template <int SEL> static __device__ __forceinline__ uint32_t cvt(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL));
  }
  static __device__ __forceinline__ f32x4_t mfma(V a, V b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Ops<__bf16> {
  typedef bf16x8_t V;
  static constexpr uint32_t kQuarterNeg2 = 0xBE80BE80u;  // -0.25 in both bf16 halves
  template <int SEL> static __device__ __forceinline__ uint32_t cvt(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
  }
  static __device__ __forceinline__ f32x4_t mfma(V a, V b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ uint32_t mark_remapped(uint32_t p, uint32_t quarter_neg2) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(short2_t, p),
                                                                __builtin_bit_cast(short2_t, quarter_neg2)));
}

struct SmArgs {
  const void* x;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* ts;
  void* y;
  int64_t n, k;
  int m;          // activation rows (<= M)
  int gpw;        // K groups per wave
  int kind, ydt;
  float m0, m1;
};

__device__ __forceinline__ void store_out(void* y, int64_t i, float v, int ydt) {
  if (ydt == kF32) ((float*)y)[i] = v;
  else if (ydt == kF16) ((_Float16*)y)[i] = (_Float16)v;
  else ((__bf16*)y)[i] = (__bf16)v;
}

// Code bytes of one lane for one tile and group: 32 / M bytes.
template <int M> struct Codes;
template <> struct Codes<1> {
  u32x4_t a, b;
  __device__ __forceinline__ void load(Rsrc r, int voff, int soff) {
    a = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNt);
    b = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, kNt);
  }
  __device__ __forceinline__ uint32_t w(int i) const { return i < 4 ? a[i] : b[i - 4]; }
};
template <> struct Codes<2> {
  u32x4_t a;
  __device__ __forceinline__ void load(Rsrc r, int voff, int soff) {
    a = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNt);
  }
  __device__ __forceinline__ uint32_t w(int i) const { return a[i]; }
};
template <> struct Codes<4> {
  u32x2_t a;
  __device__ __forceinline__ void load(Rsrc r, int voff, int soff) {
    a = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kNt);
  }
  __device__ __forceinline__ uint32_t w(int i) const { return a[i]; }
};

template <int M, int T>
struct GroupBuf {
  Codes<M> c[T];
  uint32_t s[T];
};

constexpr int kSection = 256 * 2 + 16;  // LDS bytes per K group: M x (256 / M) halves + zeros

// Weights reach the MFMA layout through LDS: a wave loads a unit of its tile
// (16 rows x 128 code bytes = 256 K elements, plus the 16 scale bytes of each
// row) with fully coalesced 16-byte loads -- each instruction covers whole
// 128-byte row segments -- writes it to a padded per-wave stage (row stride
// 144 bytes, so the MFMA-layout reads of 8 rows hit distinct banks) and reads
// each lane's slice back.  Loading the MFMA layout straight from memory would
// cover only 64 bytes of a row per instruction and double the L2 requests.
constexpr int kUnitRow = 128 + 16;              // staged code bytes per row
constexpr int kStageBytes = 16 * kUnitRow + 16 * 16;  // codes + scales of one unit

// F16S (M = 1 only): weights in the 128-element FP16-scale layout.  A unit's
// scales are one dword per row (two words, one per 128-element block), loaded
// by lanes 0..15 into the row's scale slot of the stage; a lane's D rows are
// four 16-element slots of one 128-element block, so both coefficients come
// from one word of that dword.
template <typename XT, int M, int T, int KS, bool F16S>
__global__ __launch_bounds__(64 * KS) void smallm_kernel(SmArgs a) {
  static_assert(!F16S || M == 1, "the FP16-scale layout is read for one activation row");
  typedef typename Ops<XT>::V V;
  constexpr int S = 16 / M;        // block slots per K group
  constexpr int G = 8 / M;         // MFMAs per K group
  constexpr int EPG = 256 / M;     // elements per K group
  constexpr int BPL = S / 4;       // blocks of a K group in one lane's slice
  constexpr int CB = 32 / M;       // code bytes of one lane per tile and group
  __shared__ float2 lut[256];
  __shared__ float red[KS][T][64];
  __shared__ __attribute__((aligned(16))) uint8_t stage[KS][2][T][kStageBytes];
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];  // KS * gpw sections

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, q = lane >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * (16 * T);
  const int rows_wg = (int)min((int64_t)(16 * T), a.n - row0);
  const int rcb = (int)(a.k / 2), rsb = (int)(F16S ? a.k / 64 : a.k / 16);
  const Rsrc crs = make_rsrc(a.codes + row0 * rcb, (int64_t)rows_wg * rcb);
  const Rsrc srs = make_rsrc(a.scales + row0 * rsb, (int64_t)rows_wg * rsb);
  const Rsrc xrs = make_rsrc(a.x, (int64_t)a.m * a.k * 2);
  const int nunits = (int)(a.k / 256);
  const int upw = a.gpw / M;  // units per wave
  const int u0 = wave * upw, u1 = min(nunits, u0 + upw);
  const int g0 = u0 * M, g1 = u1 * M;  // K groups of this wave
  uint8_t* xw = xs + wave * a.gpw * kSection;  // this wave's sections

  // x of this wave's groups: 32 chunks of 16 bytes per section (vector-major)
  // plus one zero chunk.  The global loads go out before any weight bytes.
  constexpr int kChunks = 33;
  constexpr int kStage = 8;  // chunks per lane held in flight (covers 15 groups)
  const int nch = (g1 - g0) * kChunks;
  u32x4_t xv[kStage];
#pragma unroll
  for (int j = 0; j < kStage; j++) {
    const int ch = lane + 64 * j, gl = ch / kChunks, r = ch % kChunks;
    const int mv = r / (EPG / 8), ee = (r % (EPG / 8)) * 8;
    const bool ok = ch < nch && r < 32 && mv < a.m;
    const int off = ok ? (int)((mv * a.k + (int64_t)(g0 + gl) * EPG + ee) * 2) : kOob;
    xv[j] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
  }

  // Coalesced unit loads: codes, lane i -> row (i >> 3) (+8 for the second
  // load), bytes 16 * (i & 7); scales, lane i -> row i >> 2, bytes 4 * (i & 3).
  const int lr = lane >> 3, lb = (lane & 7) * 16;
  int cvo0[T], cvo1[T], svo[T];
#pragma unroll
  for (int t = 0; t < T; t++) {
    cvo0[t] = 16 * t + lr < rows_wg ? (16 * t + lr) * rcb + lb : kOob;
    cvo1[t] = 16 * t + lr + 8 < rows_wg ? (16 * t + lr + 8) * rcb + lb : kOob;
    if (F16S)
      svo[t] = lane < 16 && 16 * t + lane < rows_wg ? (16 * t + lane) * rsb : kOob;
    else
      svo[t] = 16 * t + (lane >> 2) < rows_wg ? (16 * t + (lane >> 2)) * rsb + (lane & 3) * 4 : kOob;
  }
  struct UnitRegs {
    u32x4_t c0[T], c1[T];
    uint32_t s[T];
  };
  auto load_unit = [&](UnitRegs& r, int u) {
    const bool ok = u < u1;
    const int cso = ok ? u * 128 : kOob, sso = ok ? u * (F16S ? 4 : 16) : kOob;
#pragma unroll
    for (int t = 0; t < T; t++) {
      r.c0[t] = __builtin_amdgcn_raw_buffer_load_b128(crs, cvo0[t], cso, kNt);
      r.c1[t] = __builtin_amdgcn_raw_buffer_load_b128(crs, cvo1[t], cso, kNt);
      r.s[t] = __builtin_amdgcn_raw_buffer_load_b32(srs, svo[t], sso, 0);
    }
  };
  auto store_unit = [&](const UnitRegs& r, uint8_t (*st)[kStageBytes]) {
#pragma unroll
    for (int t = 0; t < T; t++) {
      *(u32x4_t*)(st[t] + lr * kUnitRow + lb) = r.c0[t];
      *(u32x4_t*)(st[t] + (lr + 8) * kUnitRow + lb) = r.c1[t];
      if (!F16S)
        *(uint32_t*)(st[t] + 16 * kUnitRow + lane * 4) = r.s[t];
      else if (lane < 16)
        *(uint32_t*)(st[t] + 16 * kUnitRow + lane * 16) = r.s[t];
    }
  };
  int xo[G];  // LDS byte offset of this lane's A fragment inside a section
  {
    const int mv = c / S, s = c % S;  // this lane's A row: vector mv, block slot s
#pragma unroll
    for (int i = 0; i < G; i++)
      xo[i] = (s == q * BPL + i / 2) ? (mv * EPG + 16 * s + 8 * (i % 2)) * 2 : 256 * 2;
  }

  UnitRegs ra, rb;
  load_unit(ra, u0);
  load_unit(rb, u0 + 1);
#pragma unroll
  for (int j = 0; j < kStage; j++) {
    const int ch = lane + 64 * j;
    if (ch < nch) *(u32x4_t*)(xw + (ch / kChunks) * kSection + (ch % kChunks) * 16) = xv[j];
  }
  for (int ch = lane + 64 * kStage; ch < nch; ch += 64) {  // long K ranges: the rest
    const int gl = ch / kChunks, r = ch % kChunks;
    const int mv = r / (EPG / 8), ee = (r % (EPG / 8)) * 8;
    const bool ok = r < 32 && mv < a.m;
    const int off = ok ? (int)((mv * a.k + (int64_t)(g0 + gl) * EPG + ee) * 2) : kOob;
    *(u32x4_t*)(xw + gl * kSection + r * 16) = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
  }
  for (int i = threadIdx.x; i < 256; i += 64 * KS) {
    float sb, sv;
    if (a.kind == kWeight) {
      sb = scale_of_byte<kWeight>(i);
      sv = special_of_byte<kWeight>(i, a.m0, a.m1);
    } else {
      sb = scale_of_byte<kAct>(i);
      sv = special_of_byte<kAct>(i, a.m0, a.m1);
    }
    lut[i] = make_float2(sb * (1.0f + 4.0f * sv), -4.0f * sb * sv);
  }
  __syncthreads();

  float acc[T];
#pragma unroll
  for (int t = 0; t < T; t++) acc[t] = 0.0f;

  // One K group (gi-th of the unit staged at st): lane (q, c) reads row c's
  // slice of every tile and the scale dword of its D rows, then G MFMA pairs
  // per tile sharing one A fragment, and the epilogue.
  auto compute_group = [&](uint8_t (*st)[kStageBytes], int gi, const uint8_t* sec) {
    uint32_t cw[T][8 / M], sw[T];
#pragma unroll
    for (int t = 0; t < T; t++) {
      const uint8_t* crow = st[t] + c * kUnitRow + gi * (128 / M) + q * CB;
      if constexpr (M == 1) {
        const u32x4_t lo = *(const u32x4_t*)crow, hi = *(const u32x4_t*)(crow + 16);
        cw[t][0] = lo[0]; cw[t][1] = lo[1]; cw[t][2] = lo[2]; cw[t][3] = lo[3];
        cw[t][4] = hi[0]; cw[t][5] = hi[1]; cw[t][6] = hi[2]; cw[t][7] = hi[3];
      } else if constexpr (M == 2) {
        const u32x4_t v = *(const u32x4_t*)crow;
        cw[t][0] = v[0]; cw[t][1] = v[1]; cw[t][2] = v[2]; cw[t][3] = v[3];
      } else {
        const u32x2_t v = *(const u32x2_t*)crow;
        cw[t][0] = v[0]; cw[t][1] = v[1];
      }
      sw[t] = F16S ? *(const uint32_t*)(st[t] + 16 * kUnitRow + c * 16)
                   : *(const uint32_t*)(st[t] + 16 * kUnitRow + c * 16 + gi * S + (4 * q) % S);
    }
    f32x4_t d0[T], d1[T];
#pragma unroll
    for (int t = 0; t < T; t++) {
      d0[t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      d1[t] = d0[t];
    }
#pragma unroll
    for (int i = 0; i < G; i++) {
      const V xa = *(const V*)(sec + xo[i]);
#pragma unroll
      for (int t = 0; t < T; t++) {
        const uint32_t w = cw[t][i];
        const u32x4_t p = {Ops<XT>::template cvt<0>(w), Ops<XT>::template cvt<1>(w),
                           Ops<XT>::template cvt<2>(w), Ops<XT>::template cvt<3>(w)};
        const u32x4_t pm = {mark_remapped(p[0], Ops<XT>::kQuarterNeg2),
                            mark_remapped(p[1], Ops<XT>::kQuarterNeg2),
                            mark_remapped(p[2], Ops<XT>::kQuarterNeg2),
                            mark_remapped(p[3], Ops<XT>::kQuarterNeg2)};
        d0[t] = Ops<XT>::mfma(xa, __builtin_bit_cast(V, p), d0[t]);
        d1[t] = Ops<XT>::mfma(xa, __builtin_bit_cast(V, pm), d1[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < T; t++) {
      if constexpr (F16S) {
        const uint32_t wd = (sw[t] >> (16 * (q >> 1))) & 0xFFFFu;  // block (4q) / 8 of the unit
        const float sb = scale_of_f16word(wd), sv = special_of_f16word(wd, a.m0, a.m1);
        const float c0 = sb * (1.0f + 4.0f * sv), c1 = -4.0f * sb * sv;
#pragma unroll
        for (int e = 0; e < 4; e++) {
          acc[t] = fmaf(d0[t][e], c0, acc[t]);
          acc[t] = fmaf(d1[t][e], c1, acc[t]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float2 f = lut[(sw[t] >> (8 * e)) & 0xFFu];
          acc[t] = fmaf(d0[t][e], f.x, acc[t]);
          acc[t] = fmaf(d1[t][e], f.y, acc[t]);
        }
      }
    }
  };

  for (int u = u0; u < u1; u += 2) {
    store_unit(ra, stage[wave][0]);
    wave_lds_sync();
    load_unit(ra, u + 2);
#pragma unroll
    for (int gi = 0; gi < M; gi++) compute_group(stage[wave][0], gi, xw + ((u - u0) * M + gi) * kSection);
    wave_lds_sync();
    if (u + 1 < u1) {
      store_unit(rb, stage[wave][1]);
      wave_lds_sync();
      load_unit(rb, u + 3);
#pragma unroll
      for (int gi = 0; gi < M; gi++) compute_group(stage[wave][1], gi, xw + ((u + 1 - u0) * M + gi) * kSection);
      wave_lds_sync();
    }
  }

#pragma unroll
  for (int t = 0; t < T; t++) red[wave][t][lane] = acc[t];
  __syncthreads();

  // Lane (q, c) of every wave holds, for weight row c of tile t, the sum over
  // the D rows 4q .. 4q+3, which all belong to vector (4q) / S.
  const float st = *a.ts;
  constexpr int QPV = S / 4;  // lane groups per vector
  for (int o = threadIdx.x; o < T * M * 16; o += 64 * KS) {
    const int t = o / (M * 16), mv = (o / 16) % M, cc = o % 16;
    const int64_t row = row0 + 16 * t + cc;
    if (mv < a.m && row < a.n) {
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < KS; w++)
#pragma unroll
        for (int j = 0; j < QPV; j++) v += red[w][t][(mv * QPV + j) * 16 + cc];
      store_out(a.y, (int64_t)mv * a.n + row, v * st, a.ydt);
    }
  }
}

struct SmPlan {
  int mt, t, ks, gpw;
  int64_t grid;
};

// Launch sizing: one 16-row tile per workgroup of KS <= 8 waves, KS the
// smallest power of two that puts about 8 waves on each CU, doubled while
// every wave still keeps >= 8 K units and the grid stays under ~16 (one row)
// or ~32 (two to four rows) waves per CU.
SmPlan plan_smallm(int64_t m, int64_t n, int64_t k, int cus, bool untrimmed = false) {
  SmPlan p;
  p.mt = m <= 1 ? 1 : m <= 2 ? 2 : 4;
  const int64_t nunits = k / 256;
  const int64_t tiles = (n + 15) / 16;
  p.t = 1;
  p.ks = 1;
  while (p.ks < 8 && tiles * p.ks < 8LL * cus && nunits / (2 * p.ks) >= 2) p.ks *= 2;
  const int64_t cap = (p.mt == 1 ? 16LL : 32LL) * cus;  // wider batches carry more LDS/epilogue work per byte
  while (p.ks < 8 && nunits / p.ks >= 8 && tiles * p.ks < cap) p.ks *= 2;
  if (untrimmed)  // the most waves per tile: up to 8, each with at least one unit
    while (p.ks < 8 && nunits / (2 * p.ks) >= 1) p.ks *= 2;
  const int64_t upw = (nunits + p.ks - 1) / p.ks;
  p.gpw = (int)(upw * p.mt);  // K groups per wave (whole units)
  p.grid = tiles;
  return p;
}

template <typename XT, int M, int T, int KS, bool F16S>
hipError_t launch_cfg(const SmArgs& a, hipStream_t stream, int64_t grid) {
  auto kern = smallm_kernel<XT, M, T, KS, F16S>;
  const size_t lds = (size_t)KS * a.gpw * kSection;
  if (lds + 2048 + KS * T * 256 + KS * 2 * T * kStageBytes > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * KS), lds, stream, a);
  return hipGetLastError();
}

template <typename XT, int M, int T, bool F16S = false>
hipError_t dispatch_ks(const SmArgs& a, const SmPlan& p, hipStream_t stream) {
  switch (p.ks) {
    case 1: return launch_cfg<XT, M, T, 1, F16S>(a, stream, p.grid);
    case 2: return launch_cfg<XT, M, T, 2, F16S>(a, stream, p.grid);
    case 4: return launch_cfg<XT, M, T, 4, F16S>(a, stream, p.grid);
    case 8: return launch_cfg<XT, M, T, 8, F16S>(a, stream, p.grid);
  }
  return hipErrorInvalidValue;
}

template <typename XT>
hipError_t dispatch(const SmArgs& a, const SmPlan& p, bool f16s, hipStream_t stream) {
  if (p.t != 1) return hipErrorInvalidValue;  // two tiles per workgroup measured slower
  if (f16s) return p.mt == 1 ? dispatch_ks<XT, 1, 1, true>(a, p, stream) : hipErrorNotSupported;
  if (p.mt == 1) return dispatch_ks<XT, 1, 1>(a, p, stream);
  if (p.mt == 2) return dispatch_ks<XT, 2, 1>(a, p, stream);
  return dispatch_ks<XT, 4, 1>(a, p, stream);
}

}  // namespace

bool smallm_supported(int64_t m, int64_t n, int64_t k) {
  // K must fill whole groups of the widest variant (256 elements for M = 1,
  // 64 for M = 4); row and x offsets must fit the 32-bit buffer offsets.
  if (m < 1 || m > 4 || n < 1 || k < 256 || k % 256 != 0) return false;
  const int mt = m <= 1 ? 1 : m <= 2 ? 2 : 4;
  if (32LL * k / 2 >= (1LL << 30)) return false;
  // x of all K groups staged in LDS next to the weight stages of up to 8 waves
  return (k / (256 / mt) + 8) * kSection <= 100 * 1024;
}

hipError_t launch_smallm(const void* x, int x_dtype, int64_t m, const PackedView& w, void* y,
                         int y_dtype, hipStream_t stream) {
  if (!smallm_supported(m, w.rows, w.cols)) return hipErrorNotSupported;
  // the default layout, or (one activation row) 128-element blocks with FP16 scales
  const bool f16s = !default_layout(w);
  if (f16s && (m != 1 || w.blog2 != 7 || w.sfmt != 1)) return hipErrorNotSupported;
  SmArgs a;
  a.x = x;
  a.codes = w.codes;
  a.scales = w.scales;
  a.ts = w.tensor_scale;
  a.y = y;
  a.n = w.rows;
  a.k = w.cols;
  a.m = (int)m;
  a.kind = w.kind;
  a.ydt = y_dtype;
  a.m0 = 6.0f + 0.5f * (float)w.off_half[0];
  a.m1 = 6.0f + 0.5f * (float)w.off_half[w.kind == kWeight ? 1 : 0];
  const SmPlan p = plan_smallm(m, w.rows, w.cols, device_cu_count(), (w.flags & kFlagUntrimmed) != 0);
  a.gpw = p.gpw;
  return x_dtype == kF16 ? dispatch<_Float16>(a, p, f16s, stream) : dispatch<__bf16>(a, p, f16s, stream);
}

}  // namespace rz
