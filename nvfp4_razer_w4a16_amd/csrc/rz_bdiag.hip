// rz_bdiag.hip -- W4A16 product for 2..8 activation rows, y[M, N] = x[M, K] * W^T,
// K a multiple of 256, on weights in the default layout (16-element blocks,
// byte scales) or in the 128-element FP16-scale layout.
//
// "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
// Remapping" (papernotes.org notes), Key design 3: the weight-only kernels
// decode the packed weights inside the kernel; "Technical Summary: RaZeR ..."
// (gist.science), §4 (moderate batches).  The pages' kernel is prior art only;
// this one is built for HBM streaming on gfx950.
//
// v_mfma_f32_16x16x32_{bf16,f16}: lane l = c + 16 q holds A row c and B column
// c at K slots 8q .. 8q+7, and D rows 4q .. 4q+3 of column c.
//   - B (weights): column c is weight row c of the wave's 16-row tile.  Lane
//     (q, c) takes bytes 32q .. 32q+31 of the row's 128 code bytes of a
//     256-element K unit (elements 64q .. 64q+63, blocks 4q .. 4q+3); MFMA i
//     (0..7) takes code dword i, i.e. elements 64q + 8i .. +7, converted by
//     the packed FP4 conversion.
//   - A (x, block-diagonal): row r = vector r % 4 (of a group of four), K-slot
//     group r / 4.  Lane (q, c) is nonzero only when c / 4 == q; it then holds
//     x[vector c % 4][64q + 8i ..].  MFMAs 2b and 2b+1 together cover block
//     4q + b of every lane group, so D[4q + e][c] is the dot of vector e with
//     block 4q + b of weight row c: one block, one scale, one special value
//     per output element, and all four of a lane's outputs share its block.
// Every block gets two products: d0 with the converted codes and d1 with the
// codes after an int16 max against -0.25, which changes only the remapped
// code (it converts to -0, the smallest int16 pattern).  The block value is
// d0 + SV * (sum of x over remapped positions) = d0 (1 + 4 SV) - 4 SV d1; a
// 256-entry LDS table holds both coefficients times the block scale, indexed
// by byte b of the lane's scale dword (dword q of the row's 16 scale bytes =
// blocks 4q .. 4q+3).  Per code dword that is 4 conversions and 4 packed
// maxes; per block and vector two fp32 FMAs.  Five to eight rows use a
// two-slot variant (eight vectors per A operand, described at the kernel).
//
// Memory: HBM streams best when each load instruction covers whole 128-byte
// row segments (16 rows x 64 bytes per instruction runs about 25 % slower), so
// a unit of a tile arrives as two 1 KiB loads of 8 rows x 128 bytes plus one
// 256-byte load of its scale bytes, with the loads of kDepth units in flight
// per wave; each wave passes a unit through its own LDS stage (chunks XOR
// swizzled by row, so both the writes and the MFMA-order reads are free of
// bank conflicts) to reach the MFMA layout.
//
// Work split: a workgroup of TR x KS waves owns TR tiles of 16 weight rows
// and all of K; wave (t, s) takes tile t and the s-th of KS contiguous K
// slices.  The waves step through their slices together: at each step the x
// of the KS units in use sits in LDS in MFMA order (one 16-byte LDS read per
// A fragment; lanes off the diagonal read a zero region placed on other
// banks), loaded two steps ahead and stored one step ahead, so it is shared by
// the TR waves of a slice without a wait on L2.  Slice partial sums meet in
// LDS at the end.
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
constexpr int kNt = 2;                  // non-temporal code loads (read once; measured faster)

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, kRsrcWord3);
}

template <typename XT> struct BdOps;
template <> struct BdOps<_Float16> {
  typedef f16x8_t V;
  static constexpr uint32_t kQuarterNeg2 = 0xB400B400u;  // -0.25 in both fp16 halves
  template <int SEL> static __device__ __forceinline__ uint32_t cvt(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL));
  }
  static __device__ __forceinline__ f32x4_t mfma(V a, V b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct BdOps<__bf16> {
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

struct BdArgs {
  const void* x;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* ts;
  void* y;
  int64_t n, k;
  int m, ydt;
  float m0, m1;
  int ups;  // K units per wave slice
};

constexpr int kStage = 16 * 128 + 16 * 16;  // one unit of a tile: codes + scale bytes

// Chunk slot of code chunk j (16 bytes) of row r in a wave's stage: the XOR
// key takes 8 distinct values over any 8 consecutive rows and, paired with the
// row parity, 16 distinct slots over 16 rows, so the reads of one chunk column
// by 8 or 16 lanes fall on distinct banks (fewer conflict cycles in the
// counters than the key (r >> 1) & 7).
__device__ __forceinline__ int stage_slot(int r, int j) { return r * 8 + (j ^ ((r & 7) ^ ((r >> 3) & 1))); }

// VG: 1 for the four-slot mapping above (up to four vectors; 2 would take a
// second group of four against the same B), or 8 for the two-slot mapping of
// five to eight vectors: A row r = vector r % 8,
// K-slot groups {2 (r / 8), 2 (r / 8) + 1}; MFMA i covers blocks 2i and
// 2i + 1, lane group q taking elements 32i + 8q .. +7 (code dword 4i + q of
// the unit), so D[4q + e][c] is vector 4 (q & 1) + e times block 2i + q / 2
// of row c.  Eight MFMAs per unit and product instead of sixteen.
//
// F16S: weights in the 128-element FP16-scale layout (the scale word's sign
// and top exponent bit carry the special value's sign and pair).  A lane's K
// slots of one unit lie in one 128-element block (four-slot: group q in block
// q / 2; two-slot: MFMAs 0..3 in block 0, 4..7 in block 1), so d0 and d1 are
// accumulated over the whole unit (four-slot) or over four MFMAs (two-slot)
// and the two coefficients, computed from the lane's scale word, are applied
// once per unit or twice.
//
// VG 16 or 32 (FP16-scale layout only, 9..32 vectors): no block diagonal.
// With one scale per 128 elements an MFMA of the two-slot K layout (MFMA i:
// elements 32i .. 32i + 31) lies in one block, so A is x itself (row r =
// vector 16t + r of x tile t) and D[4q + e][c] is vector 16t + 4q + e times
// 32 elements of block i / 4 of row c; d0 and d1 accumulate over the four
// MFMAs of a block and take the block's two coefficients once.
template <typename XT, int KIND, int VG, int TR, int KS, int D, bool F16S>
__global__ __launch_bounds__(64 * TR * KS) void bdiag_kernel(BdArgs a) {
  typedef typename BdOps<XT>::V V;
  constexpr bool DENSE = VG >= 16;                   // x tiles of 16 vectors, no diagonal
  static_assert(!DENSE || F16S, "the dense form needs one scale per 128 elements");
  constexpr bool TWO = VG == 8 || DENSE;             // the two-slot K layout
  constexpr int NG = DENSE ? VG / 16 : TWO ? 1 : VG; // A groups (x tiles) per B operand
  constexpr int NV = DENSE ? VG : TWO ? 8 : 4 * VG;  // vectors
  constexpr int NCH = DENSE ? 512 * NG : TWO ? 256 : 128 * VG;  // 16-byte x chunks per unit
  constexpr int XU = NCH * 16;                       // LDS bytes of x per K unit
  constexpr int ZB = DENSE ? 256 : XU + 256;         // zero region
  constexpr int NW = TR * KS;
  constexpr int XCH = (KS * NCH + 64 * NW - 1) / (64 * NW);  // x chunks per thread and step
  static_assert(D % 2 == 0, "the x buffers alternate with the step parity");
  __shared__ float2 lut[256];  // scale byte -> (sb (1 + 4 SV), -4 sb SV)
  __shared__ float red[KS][TR][NV][16];
  __shared__ __attribute__((aligned(16))) uint8_t stage[NW][kStage];
  // zero region, then two x buffers of KS units.  Unit chunk, four-slot:
  // (i * VG + g) * 16 + 4 q + v holds x[4g + v][elements 64q + 8i ..];
  // two-slot: (i * 4 + q) * 8 + v holds x[v][elements 32i + 8q ..];
  // dense: ((i * NG + g) * 4 + q) * 16 + v holds x[16g + v][elements 32i + 8q ..].
  __shared__ __attribute__((aligned(256))) uint8_t xl[ZB + 2 * KS * XU];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, q = lane >> 4;
  const int t = wave % TR, s = wave / TR;
  const int nunits = (int)(a.k / 256);
  const int64_t row0 = ((int64_t)blockIdx.x * TR + t) * 16;
  const int rows_w = (int)max((int64_t)0, min((int64_t)16, a.n - row0));
  const int rcb = (int)(a.k / 2), rsb = (int)(F16S ? a.k / 64 : a.k / 16);
  const Rsrc crs = make_rsrc(a.codes + (row0 < a.n ? row0 : 0) * rcb, (int64_t)rows_w * rcb);
  const Rsrc srs = make_rsrc(a.scales + (row0 < a.n ? row0 : 0) * rsb, (int64_t)rows_w * rsb);
  const Rsrc xrs = make_rsrc(a.x, (int64_t)a.m * a.k * 2);
  const int su0 = min(nunits, s * a.ups), su1 = min(nunits, su0 + a.ups);

  // Coalesced unit loads: codes, lane i -> rows i >> 3 and (i >> 3) + 8,
  // bytes 16 (i & 7); scales, lane i -> row i >> 2, bytes 4 (i & 3).
  const int lr = lane >> 3, lj = lane & 7;
  const int cvo0 = lr < rows_w ? lr * rcb + 16 * lj : kOob;
  const int cvo1 = lr + 8 < rows_w ? (lr + 8) * rcb + 16 * lj : kOob;
  // scales: byte layout, lane i -> row i >> 2, bytes 4 (i & 3) of the unit's
  // 16; FP16-scale layout, lane i < 16 -> row i, the unit's two words
  const int svo = F16S ? (lane < 16 && lane < rows_w ? lane * rsb : kOob)
                       : ((lane >> 2) < rows_w ? (lane >> 2) * rsb + 4 * (lane & 3) : kOob);
  struct Unit {
    u32x4_t c0, c1;
    uint32_t s;
  };
  auto load = [&](Unit& r, int u) {
    const bool ok = u < su1;
    const int co = ok ? u * 128 : kOob, so = ok ? u * (F16S ? 4 : 16) : kOob;
    r.c0 = __builtin_amdgcn_raw_buffer_load_b128(crs, cvo0, co, kNt);
    r.c1 = __builtin_amdgcn_raw_buffer_load_b128(crs, cvo1, co, kNt);
    r.s = __builtin_amdgcn_raw_buffer_load_b32(srs, svo, so, 0);
  };

  // x of step j (unit su0(s') + j of every slice s'): XCH chunks per thread;
  // chunks past the step, and units past a slice, load zeros (out of range)
  // and store them into the zero region, so every load has its store.
  int xoff[XCH], xdst[XCH];
  int xu0[XCH], xu1[XCH];
#pragma unroll
  for (int h = 0; h < XCH; h++) {
    const int ch = tid + h * 64 * NW;
    const int sl = ch / NCH, w = ch % NCH;
    int vec, el;
    if constexpr (DENSE) {
      vec = 16 * ((w >> 6) % NG) + (w & 15);
      el = 32 * ((w >> 6) / NG) + 8 * ((w >> 4) & 3);
    } else if constexpr (TWO) {
      vec = w & 7;
      el = 32 * (w >> 5) + 8 * ((w >> 3) & 3);
    } else {
      const int r = w >> 4;
      vec = 4 * (r % VG) + (w & 3);
      el = 64 * ((w >> 2) & 3) + 8 * (r / VG);
    }
    const bool live = ch < KS * NCH && vec < a.m;
    xoff[h] = live ? (int)(((int64_t)vec * a.k + el) * 2) : kOob;
    xdst[h] = ch < KS * NCH ? ZB + sl * XU + w * 16 : (ch % (ZB / 16)) * 16;
    xu0[h] = min(nunits, sl * a.ups);
    xu1[h] = min(nunits, xu0[h] + a.ups);
  }
  auto xload = [&](u32x4_t* v, int j) {  // (the unit offset differs per lane: voffset)
#pragma unroll
    for (int h = 0; h < XCH; h++) {
      const int u = xu0[h] + j;
      v[h] = __builtin_amdgcn_raw_buffer_load_b128(xrs, u < xu1[h] ? xoff[h] + u * 512 : kOob, 0, 0);
    }
  };
  auto xstore = [&](const u32x4_t* v, int buf) {
#pragma unroll
    for (int h = 0; h < XCH; h++) {
      const int dst = xdst[h] >= ZB ? xdst[h] + buf * KS * XU : xdst[h];
      *(u32x4_t*)(xl + dst) = v[h];
    }
  };

  // Prologue: x of steps 0 and 1, the weight loads of the first D units (in
  // the order of the steps below: the compiler counts the loads in flight by
  // position, the same on the first and later steps), the zero region and
  // the coefficient table.
  u32x4_t xv[2][XCH];
  xload(xv[0], 0);
  xload(xv[1], 1);
  Unit ring[D];
#pragma unroll
  for (int d = 0; d < D; d++) {
    __builtin_amdgcn_sched_barrier(0);
    load(ring[d], su0 + d);
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int i = tid; i < ZB / 16; i += 64 * NW) *(u32x4_t*)(xl + i * 16) = (u32x4_t){0u, 0u, 0u, 0u};
  for (int b = tid; b < 256; b += 64 * NW) {
    const float sb = scale_of_byte<KIND>(b), sv = special_of_byte<KIND>(b, a.m0, a.m1);
    lut[b] = make_float2(sb * (1.0f + 4.0f * sv), -4.0f * sb * sv);
  }
  __syncthreads();  // zero region before the x stores that may land in it
  xstore(xv[0], 0);
  __syncthreads();

  // Lanes off the diagonal read the zero region on banks away from those the
  // diagonal lanes of their group read: four-slot, group q reads banks
  // 16q .. 16q + 15 of a 256-byte window and its zeros sit at 64 ((q + 1) & 3);
  // two-slot, group q reads the (q & 1) half and its zeros sit in the other.
  const bool diag = DENSE || (TWO ? (c >> 3) == (q >> 1) : (c >> 2) == q);
  const int xa_zero = TWO ? 128 * (~q & 1) : 64 * ((q + 1) & 3);
  const int xa_diag = ZB + s * XU + (DENSE ? (16 * q + c) * 16 : TWO ? (8 * q + (c & 7)) * 16 : c * 16);
  uint8_t* st = stage[wave];
  const int w0 = stage_slot(lr, lj) * 16, w1 = stage_slot(lr + 8, lj) * 16;
  const int r0 = stage_slot(c, 2 * q) * 16, r1 = stage_slot(c, 2 * q + 1) * 16;
  float acc[NG][4];
#pragma unroll
  for (int g = 0; g < NG; g++)
#pragma unroll
    for (int e = 0; e < 4; e++) acc[g][e] = 0.0f;

  auto compute_two = [&](const Unit& r, int buf) {
    *(u32x4_t*)(st + w0) = r.c0;
    *(u32x4_t*)(st + w1) = r.c1;
    *(uint32_t*)(st + 2048 + 4 * lane) = r.s;
    wave_lds_sync();
    uint32_t cw[8];
#pragma unroll
    for (int i = 0; i < 8; i++) cw[i] = *(const uint32_t*)(st + stage_slot(c, i) * 16 + 4 * q);
    const u32x4_t sr = *(const u32x4_t*)(st + 2048 + 16 * c);
    const uint32_t sw16 = *(const uint32_t*)(st + 2048 + 4 * c);  // FP16-scale: row c's two words
    wave_lds_sync();
    const uint8_t* xb = xl + (diag ? xa_diag + buf * KS * XU : xa_zero);
    if constexpr (F16S) {
#pragma unroll
      for (int h = 0; h < 2; h++) {  // block h: MFMAs 4h .. 4h + 3
        constexpr int kFrag = DENSE ? 1024 : 512;  // bytes of the chunks of one A fragment
        f32x4_t d0[NG], d1[NG];
#pragma unroll
        for (int g = 0; g < NG; g++) {
          d0[g] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
          d1[g] = d0[g];
        }
#pragma unroll
        for (int i = 4 * h; i < 4 * h + 4; i++) {
          const uint32_t w = cw[i];
          const uint32_t p0 = BdOps<XT>::template cvt<0>(w), p1 = BdOps<XT>::template cvt<1>(w);
          const uint32_t p2 = BdOps<XT>::template cvt<2>(w), p3 = BdOps<XT>::template cvt<3>(w);
          const u32x4_t p = {p0, p1, p2, p3};
          const u32x4_t pm = {mark_remapped(p0, BdOps<XT>::kQuarterNeg2), mark_remapped(p1, BdOps<XT>::kQuarterNeg2),
                              mark_remapped(p2, BdOps<XT>::kQuarterNeg2), mark_remapped(p3, BdOps<XT>::kQuarterNeg2)};
#pragma unroll
          for (int g = 0; g < NG; g++) {
            const V xa = *(const V*)(xb + (i * NG + g) * kFrag);
            d0[g] = BdOps<XT>::mfma(xa, __builtin_bit_cast(V, p), d0[g]);
            d1[g] = BdOps<XT>::mfma(xa, __builtin_bit_cast(V, pm), d1[g]);
          }
        }
        const uint32_t wd = (sw16 >> (16 * h)) & 0xFFFFu;
        const float sb = scale_of_f16word(wd), sv = special_of_f16word(wd, a.m0, a.m1);
        const float f0 = sb * (1.0f + 4.0f * sv), f1 = -4.0f * sb * sv;
#pragma unroll
        for (int g = 0; g < NG; g++)
#pragma unroll
          for (int e = 0; e < 4; e++) {
            acc[g][e] = fmaf(d0[g][e], f0, acc[g][e]);
            acc[g][e] = fmaf(d1[g][e], f1, acc[g][e]);
          }
      }
      return;
    }
    const int sh = 8 * (q >> 1);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const uint32_t w = cw[i];
      const uint32_t p0 = BdOps<XT>::template cvt<0>(w), p1 = BdOps<XT>::template cvt<1>(w);
      const uint32_t p2 = BdOps<XT>::template cvt<2>(w), p3 = BdOps<XT>::template cvt<3>(w);
      const u32x4_t p = {p0, p1, p2, p3};
      const u32x4_t pm = {mark_remapped(p0, BdOps<XT>::kQuarterNeg2), mark_remapped(p1, BdOps<XT>::kQuarterNeg2),
                          mark_remapped(p2, BdOps<XT>::kQuarterNeg2), mark_remapped(p3, BdOps<XT>::kQuarterNeg2)};
      const V xa = *(const V*)(xb + i * 512);
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      const f32x4_t d0 = BdOps<XT>::mfma(xa, __builtin_bit_cast(V, p), z);
      const f32x4_t d1 = BdOps<XT>::mfma(xa, __builtin_bit_cast(V, pm), z);
      // block 2i + q / 2: byte 2 (i & 1) + q / 2 of scale dword i / 2
      const float2 f = lut[(sr[i >> 1] >> (16 * (i & 1) + sh)) & 0xFFu];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        acc[0][e] = fmaf(d0[e], f.x, acc[0][e]);
        acc[0][e] = fmaf(d1[e], f.y, acc[0][e]);
      }
    }
  };

  auto compute = [&](const Unit& r, int buf) {
    if constexpr (TWO) {
      compute_two(r, buf);
      return;
    }
    *(u32x4_t*)(st + w0) = r.c0;
    *(u32x4_t*)(st + w1) = r.c1;
    *(uint32_t*)(st + 2048 + 4 * lane) = r.s;
    wave_lds_sync();
    const u32x4_t lo = *(const u32x4_t*)(st + r0), hi = *(const u32x4_t*)(st + r1);
    const uint32_t sw = F16S ? *(const uint32_t*)(st + 2048 + 4 * c) : *(const uint32_t*)(st + 2048 + 16 * c + 4 * q);
    wave_lds_sync();
    const uint8_t* xb = xl + (diag ? xa_diag + buf * KS * XU : xa_zero);
    const uint32_t cw[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    if constexpr (F16S) {  // the unit's K slots of lane group q lie in block q / 2
      f32x4_t d0[NG], d1[NG];
#pragma unroll
      for (int g = 0; g < NG; g++) {
        d0[g] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        d1[g] = d0[g];
      }
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t w = cw[i];
        const uint32_t p0 = BdOps<XT>::template cvt<0>(w), p1 = BdOps<XT>::template cvt<1>(w);
        const uint32_t p2 = BdOps<XT>::template cvt<2>(w), p3 = BdOps<XT>::template cvt<3>(w);
        const u32x4_t p = {p0, p1, p2, p3};
        const u32x4_t pm = {mark_remapped(p0, BdOps<XT>::kQuarterNeg2), mark_remapped(p1, BdOps<XT>::kQuarterNeg2),
                            mark_remapped(p2, BdOps<XT>::kQuarterNeg2), mark_remapped(p3, BdOps<XT>::kQuarterNeg2)};
#pragma unroll
        for (int g = 0; g < NG; g++) {
          const V xa = *(const V*)(xb + (i * NG + g) * 256);
          d0[g] = BdOps<XT>::mfma(xa, __builtin_bit_cast(V, p), d0[g]);
          d1[g] = BdOps<XT>::mfma(xa, __builtin_bit_cast(V, pm), d1[g]);
        }
      }
      const uint32_t wd = (sw >> (16 * (q >> 1))) & 0xFFFFu;
      const float sb = scale_of_f16word(wd), sv = special_of_f16word(wd, a.m0, a.m1);
      const float f0 = sb * (1.0f + 4.0f * sv), f1 = -4.0f * sb * sv;
#pragma unroll
      for (int g = 0; g < NG; g++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          acc[g][e] = fmaf(d0[g][e], f0, acc[g][e]);
          acc[g][e] = fmaf(d1[g][e], f1, acc[g][e]);
        }
      return;
    }
#pragma unroll
    for (int b = 0; b < 4; b++) {
      f32x4_t d0[NG], d1[NG];
#pragma unroll
      for (int g = 0; g < NG; g++) {
        d0[g] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        d1[g] = d0[g];
      }
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int i = 2 * b + h;
        const uint32_t w = cw[i];
        const uint32_t p0 = BdOps<XT>::template cvt<0>(w), p1 = BdOps<XT>::template cvt<1>(w);
        const uint32_t p2 = BdOps<XT>::template cvt<2>(w), p3 = BdOps<XT>::template cvt<3>(w);
        const u32x4_t p = {p0, p1, p2, p3};
        const u32x4_t pm = {mark_remapped(p0, BdOps<XT>::kQuarterNeg2), mark_remapped(p1, BdOps<XT>::kQuarterNeg2),
                            mark_remapped(p2, BdOps<XT>::kQuarterNeg2), mark_remapped(p3, BdOps<XT>::kQuarterNeg2)};
#pragma unroll
        for (int g = 0; g < NG; g++) {
          const V xa = *(const V*)(xb + (i * NG + g) * 256);
          d0[g] = BdOps<XT>::mfma(xa, __builtin_bit_cast(V, p), d0[g]);
          d1[g] = BdOps<XT>::mfma(xa, __builtin_bit_cast(V, pm), d1[g]);
        }
      }
      const float2 f = lut[(sw >> (8 * b)) & 0xFFu];
#pragma unroll
      for (int g = 0; g < NG; g++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          acc[g][e] = fmaf(d0[g][e], f.x, acc[g][e]);
          acc[g][e] = fmaf(d1[g][e], f.y, acc[g][e]);
        }
    }
  };

  // Step j: x of step j + 2 loads, unit j of the slice is multiplied with the
  // x of buffer j & 1, the x of step j + 1 is stored into the other buffer.
  // Steps past the slice end multiply zeros (their loads were out of range).
  for (int j = 0; j < a.ups; j += D) {
#pragma unroll
    for (int d = 0; d < D; d++) {
      xload(xv[d & 1], j + d + 2);
      compute(ring[d], d & 1);
      load(ring[d], su0 + j + d + D);
      xstore(xv[(d + 1) & 1], (d + 1) & 1);
      __syncthreads();
    }
  }

  // Four-slot: lane (q, c) holds vector 4g + e over blocks 4q .. of its
  // slice; two-slot: vector 4 (q & 1) + e over blocks 2i + q / 2.  Add the
  // lane groups that share vectors, then the KS slices.
#pragma unroll
  for (int g = 0; g < NG; g++)
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float v = acc[g][e];
      if constexpr (DENSE) {  // lane group q holds vectors 16g + 4q + e
        red[s][t][16 * g + 4 * q + e][c] = v;
        continue;
      }
      if constexpr (!TWO) v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if constexpr (TWO) {
        if (q < 2) red[s][t][4 * q + e][c] = v;
      } else {
        if (q == 0) red[s][t][g * 4 + e][c] = v;
      }
    }
  __syncthreads();
  const float sc = *a.ts;
  for (int o = tid; o < TR * NV * 16; o += 64 * NW) {
    const int tt = o / (NV * 16), vec = (o / 16) % NV, cc = o % 16;
    const int64_t row = ((int64_t)blockIdx.x * TR + tt) * 16 + cc;
    if (vec < a.m && row < a.n) {
      float v = 0.0f;
#pragma unroll
      for (int ss = 0; ss < KS; ss++) v += red[ss][tt][vec][cc];
      const int64_t i = (int64_t)vec * a.n + row;
      if (a.ydt == kF32) ((float*)a.y)[i] = v * sc;
      else if (a.ydt == kF16) ((_Float16*)a.y)[i] = (_Float16)(v * sc);
      else ((__bf16*)a.y)[i] = (__bf16)(v * sc);
    }
  }
}

struct BdPlan {
  int vg, tr, ks, d, ups;
  int64_t grid;
};

// Eight waves per workgroup.  TR, the tiles per workgroup, is the largest
// power of two that still gives every CU a workgroup; the other waves split K.
// Dense x tiles (FP16-scale layout): 16 vectors take any plan (eight K slices
// of 8 KiB of x per unit still fit in LDS); 32 vectors take 8 tiles x 1 slice
// (see fp16s_supported).
BdPlan plan_bdiag(int64_t m, int64_t n, int64_t k, bool untrimmed, bool f16s) {
  BdPlan p;
  p.vg = m <= 4 ? 1 : m <= 8 ? 8 : (f16s && m <= 16) ? 16 : 32;
  const int64_t tiles = (n + 15) / 16, cus = device_cu_count();
  const int64_t nunits = k / 256;
  p.tr = 8;
  while (p.vg != 32 && p.tr > 1 && (tiles + p.tr - 1) / p.tr < cus) p.tr /= 2;
  if (untrimmed && p.vg != 32) p.tr = 1;  // the most waves per tile
  p.ks = 8 / p.tr;
  p.ups = (int)((nunits + p.ks - 1) / p.ks);
  p.d = p.ups >= 8 ? 4 : 2;
  p.grid = (tiles + p.tr - 1) / p.tr;
  return p;
}

template <typename XT, int KIND, int VG, int TR, bool F16S>
hipError_t launch_cfg(const BdArgs& a, const BdPlan& p, hipStream_t stream) {
  constexpr int KS = 8 / TR;
  if constexpr (VG == 32 && KS > 1) {  // x of two slices of 32 vectors is too much LDS
    return hipErrorNotSupported;
  } else {
  if (p.d == 4)
    hipLaunchKernelGGL((bdiag_kernel<XT, KIND, VG, TR, KS, 4, F16S>), dim3((unsigned)p.grid), dim3(64 * TR * KS),
                       0, stream, a);
  else
    hipLaunchKernelGGL((bdiag_kernel<XT, KIND, VG, TR, KS, 2, F16S>), dim3((unsigned)p.grid), dim3(64 * TR * KS),
                       0, stream, a);
  return hipGetLastError();
  }
}

template <typename XT, int KIND, int VG, bool F16S>
hipError_t dispatch_tr(const BdArgs& a, const BdPlan& p, hipStream_t stream) {
  switch (p.tr) {
    case 1: return launch_cfg<XT, KIND, VG, 1, F16S>(a, p, stream);
    case 2: return launch_cfg<XT, KIND, VG, 2, F16S>(a, p, stream);
    case 4: return launch_cfg<XT, KIND, VG, 4, F16S>(a, p, stream);
    case 8: return launch_cfg<XT, KIND, VG, 8, F16S>(a, p, stream);
  }
  return hipErrorInvalidValue;
}

template <typename XT, int KIND, bool F16S = false>
hipError_t dispatch_vg(const BdArgs& a, const BdPlan& p, hipStream_t stream) {
  if (p.vg == 1) return dispatch_tr<XT, KIND, 1, F16S>(a, p, stream);
  if (p.vg == 8) return dispatch_tr<XT, KIND, 8, F16S>(a, p, stream);
  if constexpr (F16S) {
    if (p.vg == 16) return dispatch_tr<XT, KIND, 16, F16S>(a, p, stream);
    if (p.vg == 32) return dispatch_tr<XT, KIND, 32, F16S>(a, p, stream);
  }
  return hipErrorNotSupported;
}

}  // namespace

bool bdiag_supported(int64_t m, int64_t n, int64_t k) {
  return m >= 2 && m <= 8 && n >= 1 && n < (1LL << 31) && k >= 256 && k % 256 == 0 && k < (1LL << 24);
}

// FP16-scale layout: 2..16 rows, and 17..32 rows on weights of at least
// 4 x 16 rows per CU (their plan puts 8 tiles in a workgroup).
bool fp16s_supported(int64_t m, int64_t n, int64_t k) {
  if (m > 16 && (n + 15) / 16 < 4LL * device_cu_count()) return false;
  return m >= 2 && m <= 32 && n >= 1 && n < (1LL << 31) && k >= 256 && k % 256 == 0 && k < (1LL << 24);
}

hipError_t launch_bdiag(const void* x, int x_dtype, int64_t m, const PackedView& w, void* y, int y_dtype,
                        hipStream_t stream) {
  const bool f16s = w.blog2 == 7 && w.sfmt == 1 && w.kind == kWeight;
  if (!(default_layout(w) || f16s)) return hipErrorNotSupported;
  if (f16s ? !fp16s_supported(m, w.rows, w.cols) : !bdiag_supported(m, w.rows, w.cols)) return hipErrorNotSupported;
  if (x_dtype != kF16 && x_dtype != kBF16) return hipErrorInvalidValue;
  const BdPlan p = plan_bdiag(m, w.rows, w.cols, (w.flags & kFlagUntrimmed) != 0, f16s);
  BdArgs a;
  a.x = x;
  a.codes = w.codes;
  a.scales = w.scales;
  a.ts = w.tensor_scale;
  a.y = y;
  a.n = w.rows;
  a.k = w.cols;
  a.m = (int)m;
  a.ydt = y_dtype;
  a.m0 = 6.0f + 0.5f * (float)w.off_half[0];
  a.m1 = 6.0f + 0.5f * (float)w.off_half[w.kind == kWeight ? 1 : 0];
  a.ups = p.ups;
  if (f16s)
    return x_dtype == kBF16 ? dispatch_vg<__bf16, kWeight, true>(a, p, stream)
                            : dispatch_vg<_Float16, kWeight, true>(a, p, stream);
  if (x_dtype == kBF16)
    return w.kind == kWeight ? dispatch_vg<__bf16, kWeight>(a, p, stream) : dispatch_vg<__bf16, kAct>(a, p, stream);
  return w.kind == kWeight ? dispatch_vg<_Float16, kWeight>(a, p, stream) : dispatch_vg<_Float16, kAct>(a, p, stream);
}

}  // namespace rz
