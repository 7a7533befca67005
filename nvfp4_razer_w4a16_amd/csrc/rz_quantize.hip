// rz_quantize.hip -- RaZeR encoder for gfx950: tensor amax pass + block encode.
//
// Method: "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
// Remapping" (papernotes.org notes), Overall framework and Key designs 1-2;
// "Technical Summary: RaZeR ..." (gist.science), §2.1-2.2.
//
// Pass 1 (amax_partial_kernel): each workgroup reduces |x| over a grid-stride
// slice with 128-bit loads and writes one partial maximum (as fp32 bits; NaN
// and Inf sort above every finite value) to the workspace.  No atomics, so
// the workspace needs no clearing and the pass can be graph-captured.
// Pass 2 (encode_kernel): every workgroup folds the partials into the tensor
// amax, then encodes 16-element blocks, one block per lane (64 consecutive
// blocks per wave and step, read with contiguous loads through LDS):
//   st = amax / (6 * S_MAX); sb = nearest-even(S_MAX * amax_b / amax) on the
//   E3M3 / E4M3 grid; y = x * (1 / (sb * st)); FP4 nearest-even codes; the
//   special value whose block squared error is lowest replaces the redundant
//   -0 code.  All fp32 steps are single IEEE operations in a fixed order
//   (this file is compiled with -ffp-contract=off), so the bytes are
//   reproducible on any IEEE machine.
//
// Exact candidate comparison: moving element y (|y| = a) from its FP4 rounding
// q to the special value M changes the block squared error by
// (M - q)(M + q - 2a).  Only elements inside M's window (closer to M than to
// either FP4 neighbour) move, and for them q is the grid point just below or
// just above M.  With a power of two 2^s (s = 21, or 20 when the window starts
// at 4 or above), V = 2^s (M + q) - 2^(s+1) a is an integer (a > 2 is a
// multiple of 2^-22, a >= 4 of 2^-21) with |V| < 2^23, one fma computes it
// exactly, and the change is (2M - 2q) V / 2^(s+1).  The products fit the
// 24-bit multiplier and 16 of them fit int32, so every candidate's change is
// summed exactly and the argmin (ties to the lowest candidate index) never
// depends on rounding or summation order.  The bound on V needs every |y| of
// the block below kFastCap, which fails only for blocks whose tensor scale is
// subnormal; those blocks take the same comparison in int64 with
// A = a * 2^22: (2M - 2q) * ((2M + 2q) * 2^21 - 2A).
#include "rz_device.h"
#include "rz_launch.h"

#include <math.h>

#include <mutex>
#include <type_traits>

namespace rz {

Candidate make_candidate(int off_half) {
  static const double kGrid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  const double M = 6.0 + off_half / 2.0;
  Candidate c;
  c.mag = (float)M;
  c.mag_x2 = 12 + off_half;
  bool on_grid = false;
  double below = 0.0, above = INFINITY;
  for (double g : kGrid) {
    if (g == M) on_grid = true;
    if (g < M && g > below) below = g;
    if (g > M && g < above) above = g;
  }
  if (on_grid) {
    c.lo = c.hi = 0.0f;  // an FP4 value never wins (a tie keeps the FP4 code)
  } else {
    c.lo = (float)((below + M) / 2.0);  // exact: quarter-integers
    c.hi = std::isinf(above) ? INFINITY : (float)((M + above) / 2.0);
  }
  return c;
}

size_t quantize_ws_bytes() { return kAmaxMaxPartials * sizeof(uint32_t); }

// Per candidate pair, for the int32 search (see the header comment).
struct PairFast {
  float lo, hi;     // window: lo < |y| < hi moves to M (lo = hi = 0: M is an FP4 value)
  float thr;        // |y| >= thr rounds to the grid point above M (ties to the even code)
  float klo, khi;   // 2^s (M + q) for q below / above M
  float ascale;     // -2^(s+1)
  int ddlo, ddhi;   // 2M - 2q for q below / above M (|.| <= 7)
  int shift;        // 21 - s: brings the pair's sums to the common scale
};

struct EncodeParams {
  float lo[2], hi[2];
  int mag_x2[2];
  PairFast f[2];
  int remap;
  // Activations whose candidate M is the midpoint of its FP4 neighbours (M =
  // 2.5, 3.5 or 5, half-gap h = 0.5, 0.5, 1): the midpoint search below.
  int sym = 0;
  float sym_m = 0.0f, sym_h = 0.0f;
};

constexpr float kFastCap = 10.0f;

static PairFast make_pair_fast(int off_half) {
  static const double kGrid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  const Candidate c = make_candidate(off_half);
  PairFast f{};
  if (c.hi == 0.0f) return f;  // M on the FP4 grid: no element ever moves
  const double M = 6.0 + off_half / 2.0;
  int i = 0;  // index of the grid point just below M
  while (i + 1 < 8 && kGrid[i + 1] < M) i++;
  const double below = kGrid[i];
  const bool top = i == 7;  // M above 6: every moved element rounds to 6
  const double above = top ? below : kGrid[i + 1];
  const int s = c.lo >= 4.0f ? 20 : 21;
  f.lo = c.lo;
  f.hi = c.hi;
  if (top) {
    f.thr = INFINITY;
  } else {
    const float mid = (float)((below + above) / 2.0);
    // a tie rounds to the even grid index: up when i + 1 is even
    f.thr = ((i + 1) % 2 == 0) ? mid : nextafterf(mid, INFINITY);
  }
  f.klo = (float)std::ldexp(M + below, s);
  f.khi = (float)std::ldexp(M + above, s);
  f.ascale = (float)-std::ldexp(1.0, s + 1);
  f.ddlo = (int)(2.0 * (M - below));
  f.ddhi = (int)(2.0 * (M - above));
  f.shift = 21 - s;
  return f;
}

// ---- pass 1: partial tensor amax ---------------------------------------------
// |x| as fp32 bit patterns: unsigned order equals magnitude order, and NaN/Inf
// (>= 0x7F800000) sort above every finite value.
template <typename T> __device__ __forceinline__ uint32_t absbits_max(uint4 v);

template <> __device__ __forceinline__ uint32_t absbits_max<float>(uint4 v) {
  return max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
}
template <> __device__ __forceinline__ uint32_t absbits_max<__bf16>(uint4 v) {
  uint32_t m = 0;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; i++) m = max(m, max(w[i] & 0x7FFF0000u, (w[i] << 16) & 0x7FFF0000u));
  return m;
}
// fp16: reduce 15-bit magnitudes (monotone in value), widened to fp32 later.
template <> __device__ __forceinline__ uint32_t absbits_max<_Float16>(uint4 v) {
  uint32_t m = 0;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; i++) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  return m;
}

template <typename T> __device__ __forceinline__ uint32_t absbits_finish(uint32_t m) { return m; }
template <> __device__ __forceinline__ uint32_t absbits_finish<_Float16>(uint32_t m) {
  return f2u((float)__builtin_bit_cast(_Float16, (uint16_t)m));
}

// KEEP: default-policy loads, so that a tensor that fits the memory-side cache
// is still there for the encode pass, which reads it again right after this
// one; larger tensors are streamed (non-temporal loads).
template <typename T, bool KEEP>
__global__ __launch_bounds__(256) void amax_partial_kernel(const uint4* __restrict__ x, int64_t nvec,
                                                           uint32_t* __restrict__ partial) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  auto ld = [&](int64_t j) { return KEEP ? x[j] : load_nt16(x + j); };
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    uint4 a = ld(i);
    uint4 b = ld(i + stride);
    uint4 c = ld(i + 2 * stride);
    uint4 d = ld(i + 3 * stride);
    m = max(m, max(max(absbits_max<T>(a), absbits_max<T>(b)), max(absbits_max<T>(c), absbits_max<T>(d))));
  }
  for (; i < nvec; i += stride) m = max(m, absbits_max<T>(x[i]));
  m = wave_max_u32(absbits_finish<T>(m));
  __shared__ uint32_t sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = max(max(sm[0], sm[1]), max(sm[2], sm[3]));
}

// Tensors up to this size are read with default-policy loads in the amax pass
// (the 256 MB memory-side cache then still holds them for the encode pass).
constexpr int64_t kAmaxKeepBytes = 128ll << 20;

// Workgroups of the amax pass: two per CU (eight waves), each with four
// 16-byte loads per thread in flight.  Measured against one workgroup per 1024
// 16-byte vectors up to 1024 workgroups: X [4096, 8192] bf16 encodes in 30.9
// against 32.7 us, W [28672, 8192] fp32 in 0.337 against 0.369 ms (256 or
// 1024 workgroups, or two loads per thread in flight, are slower).
static int64_t amax_grid(int64_t nvec) {
  int64_t g = (nvec + 4 * 256 - 1) / (4 * 256);
  const int64_t cap = 2LL * device_cu_count();
  if (g > cap) g = cap;
  if (g > kAmaxMaxPartials) g = kAmaxMaxPartials;
  return g < 1 ? 1 : g;
}

template <typename T>
static void launch_amax_partial(dim3 grid, hipStream_t stream, const uint4* x, int64_t nvec, uint32_t* partial) {
  if (nvec * 16 <= kAmaxKeepBytes)
    hipLaunchKernelGGL((amax_partial_kernel<T, true>), grid, dim3(256), 0, stream, x, nvec, partial);
  else
    hipLaunchKernelGGL((amax_partial_kernel<T, false>), grid, dim3(256), 0, stream, x, nvec, partial);
}

// ---- pass 2: block encode ----------------------------------------------------
// Nearest-even block-scale code for v >= 0, saturating at the format maximum.
// Normal range: keep 3 mantissa bits of the fp32 value with a round-to-even
// carry; subnormal range: round v / quantum to an integer (v_rndne_f32).  The
// subnormal result 8 is exactly the smallest normal code, so both ranges join.
template <int KIND> __device__ __forceinline__ uint32_t round_scale(float v) {
  constexpr float kMax = KIND == kWeight ? 30.0f : 448.0f;
  constexpr float kNormMin = KIND == kWeight ? 0.25f : 0.015625f;
  constexpr float kSubInv = KIND == kWeight ? 32.0f : 512.0f;
  constexpr int kBias = KIND == kWeight ? 3 : 7;
  constexpr uint32_t kMaxCode = KIND == kWeight ? 63u : 126u;
  if (v >= kMax) return kMaxCode;
  if (v < kNormMin) return (uint32_t)__builtin_rintf(v * kSubInv);
  uint32_t b = f2u(v);
  b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;
  uint32_t code = ((uint32_t)((int)(b >> 23) - 127 + kBias) << 3) | ((b >> 20) & 7u);
  return min(code, kMaxCode);
}

// round_scale for a block: sb_real = S_MAX * amax_b / amax never exceeds S_MAX.
// For activations (OCP E4M3) the gfx950 fp32 -> fp8 conversion (scale 1)
// gives the same code as round_scale on every fp32 value in [0, 448]
// (nearest-even in the normal and subnormal ranges alike; checked on all of
// them); weights (E3M3, no hardware format) keep the software rounding.
template <int KIND> __device__ __forceinline__ uint32_t round_scale_block(float v) {
  if constexpr (KIND == kAct) {
    typedef short v2i16 __attribute__((ext_vector_type(2)));
    const v2i16 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2i16{0, 0}, v, 0.0f, 1.0f, false);
    return (uint32_t)(uint16_t)r.x & 0xFFu;
  } else {
    return round_scale<KIND>(v);
  }
}

template <int KIND> __device__ __forceinline__ float scale_of_code(uint32_t code) {
  return scale_of_byte<KIND>(code);
}

// d * v + c on the 24-bit multiplier (v_mad_i32_i24 reads the low 24 bits of
// d and v, sign-extended).  Written out because the compiler otherwise spends a
// mask or sign-extension on an operand whose range it cannot see.
__device__ __forceinline__ int mad_i24(int d, int v, int c) {
  int r;
  asm("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(r) : "v"(d), "v"(v), "v"(c));
  return r;
}

// Fast exact search (int32 sums, see the header comment) and the remap of the
// chosen candidate's elements to code 0b1000.  Returns the candidate index.
template <int KIND>
__device__ __forceinline__ uint32_t search_fast(const float (&y)[16], float ymax, uint32_t (&w)[2],
                                                const EncodeParams& prm) {
  constexpr int kPairs = KIND == kWeight ? 2 : 1;
  int pos[kPairs], neg[kPairs];  // summed changes of the +M and -M candidates
  uint32_t bits[kPairs];         // bit j: element j is inside the pair's window
#pragma unroll
  for (int p = 0; p < kPairs; p++) pos[p] = neg[p] = 0, bits[p] = 0u;
  // Midpoint candidate (activations): with u = |y| - M and h half the gap
  // between M's FP4 neighbours, an element moves iff |u| < h / 2, and its
  // change is -h (h - 2|u|) whichever neighbour it rounds to.  So
  // D = sum over the block of sign(y) * max(h - 2|u|, 0) orders the two
  // candidates: +M loses (sel 1) iff D < 0.  Near the window a is within a
  // factor of two of M, so u is exact, and h - 2|u| is a multiple of 2^-20
  // (a >= 4) or 2^-21 (a >= 2) of magnitude at most 1, so every partial sum
  // of 16 of them is exact in fp32; away from the window the term is 0
  // whatever the rounding.  Five operations per element instead of the
  // integer form's window tests, fma, conversion and multiply-add.
  // h <= 1, so max(h - 2|u|, 0) is the fma with its result clamped to [0, 1].
  // The window marks go straight to their nibbles (bit 4i of dword i / 8).
  bool sym_done = false;
  uint32_t sym_sel = 0u;
  uint32_t sym_nib[2] = {0u, 0u};
  if constexpr (kPairs == 1) {
    if (prm.sym) {
      sym_done = true;
      if (ymax > prm.lo[0]) {
        float dsum;
        uint32_t tb[16];
#pragma unroll
        for (int j = 15; j >= 0; j--) {
          const float u = fabsf(y[j]) - prm.sym_m;
          float t;
          asm("v_fma_f32 %0, |%1|, -2.0, %2 clamp" : "=v"(t) : "v"(u), "v"(prm.sym_h));
          tb[j] = __builtin_bit_cast(uint32_t, t);
          const float term = __builtin_bit_cast(float, tb[j] | (__builtin_bit_cast(uint32_t, y[j]) & 0x80000000u));
          dsum = j == 15 ? term : dsum + term;
        }
        // Window marks, two elements per step: a nonzero t is at least 2^-21,
        // so its upper 16 bits are nonzero.  Elements i and i + 4 of a code
        // dword have their upper halves gathered into one register, each half
        // is clamped to 0 / 1, and one shift-or puts them at bits 4i and
        // 4i + 16 (asm: the compiler would turn these into compares and selects).
        const uint32_t ones = 0x00010001u;
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const uint32_t hi2 = __builtin_amdgcn_perm(tb[8 * h + i + 4], tb[8 * h + i], 0x07060302u);
            uint32_t mk;
            asm("v_pk_min_u16 %0, %1, %2" : "=v"(mk) : "v"(hi2), "v"(ones));
            asm("v_lshl_or_b32 %0, %1, %2, %3" : "=v"(sym_nib[h]) : "v"(mk), "i"(4 * i), "v"(sym_nib[h]));
          }
        sym_sel = dsum < 0.0f ? 1u : 0u;
      }
    }
  }
#pragma unroll
  for (int p = 0; p < kPairs; p++) {
    if (sym_done) continue;
    const PairFast& f = prm.f[p];
    const int dlo = f.ddlo, dhi = f.ddhi;
    // ymax = max |y| of the block exactly (rounding is monotone): at or below
    // the window no element moves, and a wave whose lanes all are skips the
    // pair (the usual case for a pair above 6, reachable only from blocks
    // whose scale rounded down to a subnormal code)
    if (!(ymax > f.lo && f.hi > f.lo)) continue;
#pragma unroll
    for (int j = 15; j >= 0; j--) {
      const float a = fabsf(y[j]);
      const bool in = a > f.lo && a < f.hi;
      const bool up = a >= f.thr;
      const float k = up ? f.khi : f.klo;
      const int d = in ? (up ? dhi : dlo) : 0;
      if constexpr (kPairs == 1) {
        // one sum: sign(y) * V from the fma with sign(y) * 2^s (M + q), so
        // pos[0] accumulates (+M change) - (-M change)
        const float ks = __builtin_bit_cast(
            float, __builtin_bit_cast(uint32_t, k) | (__builtin_bit_cast(uint32_t, y[j]) & 0x80000000u));
        pos[p] = mad_i24(d, (int)__builtin_fmaf(y[j], f.ascale, ks), pos[p]);
      } else {
        const int t = mad_i24(d, (int)__builtin_fmaf(a, f.ascale, k), 0);
        pos[p] += t;  // all moved elements here; the -M part is taken out below
        neg[p] += y[j] < 0.0f ? t : 0;
      }
      bits[p] = bits[p] + bits[p] + (in ? 1u : 0u);
    }
    if constexpr (kPairs == 2) pos[p] -= neg[p];
  }
  // candidates +M0, -M0 (, +M1, -M1): lowest change wins, ties to the lower index
  uint32_t sel = 0u;
  if constexpr (kPairs == 1) {
    sel = sym_done ? sym_sel : (pos[0] > 0 ? 1u : 0u);  // (+M change) > (-M change)
  } else {
    int best = pos[0] * (1 << prm.f[0].shift);
    const int c1 = neg[0] * (1 << prm.f[0].shift);
    const int c2 = pos[1] * (1 << prm.f[1].shift);
    const int c3 = neg[1] * (1 << prm.f[1].shift);
    if (c1 < best) best = c1, sel = 1u;
    if (c2 < best) best = c2, sel = 2u;
    if (c3 < best) best = c3, sel = 3u;
  }
  // elements of the chosen pair's window whose sign matches the candidate
  // (the sign is bit 3 of their nonzero FP4 code) become code 0b1000
  const uint32_t b = (kPairs == 2 && (sel >> 1)) ? bits[kPairs - 1] : bits[0];
  const uint32_t keep = (sel & 1u) ? 0u : 0x11111111u;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    uint32_t x;
    if (sym_done) {
      x = sym_nib[h];
    } else {
      x = (b >> (8 * h)) & 0xFFu;  // element 8h + i -> bit 4i
      x = (x | (x << 12)) & 0x000F000Fu;
      x = (x | (x << 6)) & 0x03030303u;
      x = (x | (x << 3)) & 0x11111111u;
    }
    const uint32_t hit = x & ((w[h] >> 3) ^ keep);
    // 15 per hit nibble, as a shift and a subtract (written as asm: the
    // compiler would fold them into a quarter-rate 32-bit multiply)
    uint32_t nib;
    asm("v_sub_u32 %0, %1, %2" : "=v"(nib) : "v"(hit << 4), "v"(hit));
    w[h] = (w[h] & ~nib) | (hit << 3);
  }
  return sel;
}

// FP4 codes with the gfx950 conversion: nearest on the E2M1 grid, ties to the
// even code (0.25, 1.25, 2.5, 5 go down; 0.75, 1.75, 3.5 go up), saturating at
// 6, sign in bit 3.  A negative value that rounds to zero comes out as 0b1000
// and is cleared to +0.
__device__ __forceinline__ void fp4_pack16(const float (&y)[16], uint32_t (&w)[2]) {
#pragma unroll
  for (int h = 0; h < 2; h++) {
    w[h] = 0u;
    w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], y[8 * h + 0], y[8 * h + 1], 1.0f, 0);
    w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], y[8 * h + 2], y[8 * h + 3], 1.0f, 1);
    w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], y[8 * h + 4], y[8 * h + 5], 1.0f, 2);
    w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], y[8 * h + 6], y[8 * h + 7], 1.0f, 3);
    const uint32_t nz = (w[h] & 0x77777777u) + 0x77777777u;  // bit 3: magnitude != 0
    w[h] &= ~(~nz & 0x88888888u);                            // -0 -> +0
  }
}

// 1 / (sb * st) for every block-scale code (sb * st, then one IEEE division:
// the same two operations a block would do itself), built once per workgroup.
template <int KIND> constexpr int kScaleCodes = KIND == kWeight ? 64 : 128;
template <int KIND>
__device__ __forceinline__ void build_rcp_table(float* rtab, float st) {
  for (int c = threadIdx.x; c < kScaleCodes<KIND>; c += blockDim.x)
    rtab[c] = 1.0f / (scale_of_code<KIND>((uint32_t)c) * st);
}

// amax_b / amax, the IEEE fp32 quotient.  With FASTDIV (16-bit inputs, amax in
// [2^-60, 2^60]) it is computed from rinv = 1 / amax (one IEEE division per
// kernel) by Markstein's correction: q0 = amax_b * rinv, e = amax_b - q0 * amax
// (exact in an fma), q = q0 + e * rinv.  Markstein's theorem gives the correctly
// rounded quotient for a correctly rounded reciprocal, a faithful q0 and no
// underflow; for 8- and 11-bit significands it was also checked on every pair
// (a CPU model against exact rationals).  Where the operands leave the normal
// range the quotient is far below 2^-18, whose scale code is 0 either way.
template <bool FASTDIV>
__device__ __forceinline__ float block_ratio(float amax_b, float amax, float rinv) {
  if constexpr (FASTDIV) {
    const float q0 = amax_b * rinv;
    const float e = __builtin_fmaf(-q0, amax, amax_b);
    return __builtin_fmaf(e, rinv, q0);
  } else {
    return amax_b / amax;
  }
}

template <int KIND, bool FASTDIV = false>
__device__ __forceinline__ void encode_block(const float (&xf)[16], float amax, float rinv, const float* rtab,
                                             const EncodeParams& prm, uint2& cw, uint32_t& sbyte) {
  constexpr float kSMax = KIND == kWeight ? 30.0f : 448.0f;
  constexpr int kPairs = KIND == kWeight ? 2 : 1;
  cw = make_uint2(0u, 0u);
  sbyte = 0u;
  float amax_b = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; j++) amax_b = fmaxf(amax_b, fabsf(xf[j]));
  const float r = block_ratio<FASTDIV>(amax_b, amax, rinv);
  const float sb_real = r * kSMax;
  const uint32_t scode = round_scale_block<KIND>(sb_real);
  if (scode == 0u) return;  // block underflows to zero
  const float rcp = rtab[scode];  // 1 / (sb * st)
  if (!(rcp < INFINITY)) return;  // scale product underflowed: zero block

  float y[16];
#pragma unroll
  for (int j = 0; j < 16; j++) y[j] = xf[j] * rcp;
  uint32_t w[2];
  fp4_pack16(y, w);
  uint32_t sel = 0u;
  const float ymax = amax_b * rcp;
  if (prm.remap && ymax < kFastCap) {
    sel = search_fast<KIND>(y, ymax, w, prm);
  } else if (prm.remap) {
    long long acc[2 * kPairs];
#pragma unroll
    for (int c = 0; c < 2 * kPairs; c++) acc[c] = 0;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const uint32_t c = (w[j >> 3] >> (4 * (j & 7))) & 15u;
      const uint32_t nj = c >> 3;  // moved elements have |y| > 2, so the code keeps the sign
      const float aj = fabsf(y[j]);
      const int q2 = (int)fp4_mag_x2(c & 7u);
      const int a2 = 2 * (int)(aj * 4194304.0f);  // 2 * a * 2^22 (exact when it matters)
#pragma unroll
      for (int p = 0; p < kPairs; p++) {
        const bool in = aj > prm.lo[p] && aj < prm.hi[p];
        const int dd = prm.mag_x2[p] - q2;
        const int ee = ((prm.mag_x2[p] + q2) << 21) - a2;
        const int dpos = (in && !nj) ? dd : 0;
        const int dneg = (in && nj) ? dd : 0;
        acc[2 * p] += (long long)dpos * (long long)ee;
        acc[2 * p + 1] += (long long)dneg * (long long)ee;
      }
    }
    long long best = acc[0];
#pragma unroll
    for (int c = 1; c < 2 * kPairs; c++)
      if (acc[c] < best) {
        best = acc[c];
        sel = (uint32_t)c;
      }
    const int p = (int)(sel >> 1);
    const uint32_t sneg = sel & 1u;
    const float lo = prm.lo[p], hi = prm.hi[p];
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const uint32_t sh = 4 * (j & 7);
      const uint32_t c = (w[j >> 3] >> sh) & 15u;
      const float aj = fabsf(y[j]);
      const bool hit = aj > lo && aj < hi && (c >> 3) == sneg;
      w[j >> 3] ^= hit ? ((c ^ 8u) << sh) : 0u;  // the special value's code
    }
  }
  cw = make_uint2(w[0], w[1]);
  sbyte = (KIND == kWeight) ? (((sel & 1u) << 7) | ((sel >> 1) << 6) | scode) : ((sel << 7) | scode);
}

// ---- Four Over Six baseline (plain FP4, adaptive block scale) ----------------
// Page "Four Over Six: More Accurate NVFP4 Quantization with Adaptive Block
// Scaling", technical framework and key innovation: a block may be scaled so
// that its maximum maps to 4 instead of 6.  Each block is encoded twice as
// plain FP4, at the nearest scale code to sb_real (max -> 6) and to
// 1.5 * sb_real (max -> 4), and keeps the encoding whose squared error in real
// units is smaller; a tie keeps max -> 6.

// Squared error of a plain-FP4 block: sum over j in order of
// (x_j - value_j * sb * st)^2 in fp64.  value * sb * st is exact in fp64; the
// difference, the square and each partial sum round once each, so no
// contraction into fused multiply-adds.
__device__ __forceinline__ double plain_block_sse(const float (&xf)[16], const uint32_t (&w)[2],
                                                  float sb, float st, double sse = 0.0) {
#pragma clang fp contract(off)
  const double s = (double)sb * (double)st;
#pragma unroll
  for (int j = 0; j < 16; j++) {
    const uint32_t c = (w[j >> 3] >> (4 * (j & 7))) & 15u;
    const double v = 0.5 * (double)fp4_mag_x2(c & 7u);
    const double q = (c & 8u) ? -(v * s) : v * s;
    const double e = (double)xf[j] - q;
    sse = sse + e * e;
  }
  return sse;
}

// One plain-FP4 encoding at real block scale sb_real; returns the scale code
// (0: the block is stored as zero) and the block's squared error.
template <int KIND>
__device__ __forceinline__ uint32_t plain_at_scale(const float (&xf)[16], float sb_real, float st,
                                                   uint32_t (&w)[2], double& sse) {
  w[0] = 0u;
  w[1] = 0u;
  uint32_t scode = round_scale<KIND>(sb_real);
  float sb = 0.0f;
  if (scode != 0u) {
    sb = scale_of_code<KIND>(scode);
    const float d = sb * st;
    const float rcp = 1.0f / d;
    if (rcp < INFINITY) {
      float y[16];
#pragma unroll
      for (int j = 0; j < 16; j++) y[j] = xf[j] * rcp;
      fp4_pack16(y, w);
    } else {
      scode = 0u;
      sb = 0.0f;
    }
  }
  sse = plain_block_sse(xf, w, sb, st);
  return scode;
}

template <int KIND>
__device__ __forceinline__ void encode_block_fos(const float (&xf)[16], float amax, float st,
                                                 uint2& cw, uint32_t& sbyte) {
  constexpr float kSMax = KIND == kWeight ? 30.0f : 448.0f;
  float amax_b = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; j++) amax_b = fmaxf(amax_b, fabsf(xf[j]));
  const float r = amax_b / amax;
  const float sb_real = r * kSMax;
  uint32_t w6[2], w4[2];
  double e6, e4;
  const uint32_t c6 = plain_at_scale<KIND>(xf, sb_real, st, w6, e6);
  const uint32_t c4 = plain_at_scale<KIND>(xf, sb_real * 1.5f, st, w4, e4);
  const bool four = e4 < e6;
  cw = four ? make_uint2(w4[0], w4[1]) : make_uint2(w6[0], w6[1]);
  sbyte = four ? c4 : c6;
}

// ---- RaZeR with rescaled large special values --------------------------------
// A reading of "RaZeR ..." (papernotes.org notes), Training strategy: the best
// weight pairs it reports include +/-7, +/-8 and +/-9, which a block scaled
// so that its maximum maps to 6 almost never reaches.  Each candidate v is
// tried on its own: one with |v| > 6 at the block scale nearest to
// (sb_real * 6) / |v| (the block maximum then maps to |v|), the others at the
// usual scale; its elements strictly nearer to v than to their FP4 rounding
// take the special-value code.  The block keeps the encoding with the smallest
// squared error in real units, summed in fp64 in element order (every decoded
// value * sb * st is exact in fp64; the difference, the square and each
// partial sum round once), ties to the lowest candidate index.  A candidate
// whose scale code or scale product underflows stores the block as zero.
template <int KIND>
__device__ __forceinline__ void encode_block_rescale(const float (&xf)[16], float amax, float st,
                                                     const float* rtab, const EncodeParams& prm, uint2& cw,
                                                     uint32_t& sbyte) {
#pragma clang fp contract(off)
  constexpr float kSMax = KIND == kWeight ? 30.0f : 448.0f;
  constexpr int kCand = KIND == kWeight ? 4 : 2;
  float amax_b = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; j++) amax_b = fmaxf(amax_b, fabsf(xf[j]));
  const float r = amax_b / amax;
  const float sb_real = r * kSMax;
  double best = 0.0;
  uint32_t bsel = 0u, bcode = 0u, bw0 = 0u, bw1 = 0u;
#pragma unroll
  for (int c = 0; c < kCand; c++) {
    const int p = c >> 1;
    const uint32_t neg = (uint32_t)(c & 1);
    const float mag = 0.5f * (float)prm.mag_x2[p];
    const float sbr = mag > 6.0f ? (sb_real * 6.0f) / mag : sb_real;
    uint32_t scode = round_scale_block<KIND>(sbr);
    uint32_t w[2] = {0u, 0u};
    const float rcp = scode ? rtab[scode] : 0.0f;
    if (!(rcp < INFINITY)) scode = 0u;
    float y[16];
#pragma unroll
    for (int j = 0; j < 16; j++) y[j] = xf[j] * rcp;
    if (scode) {
      fp4_pack16(y, w);
      const float lo = prm.lo[p], hi = prm.hi[p];
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const uint32_t sh = 4 * (j & 7);
        const uint32_t code = (w[j >> 3] >> sh) & 15u;
        const float aj = fabsf(y[j]);
        // a moved element lies above 2, so its FP4 code carries the sign
        const bool hit = aj > lo && aj < hi && (code >> 3) == neg;
        w[j >> 3] ^= hit ? ((code ^ 8u) << sh) : 0u;
      }
    }
    const double sbst = scode ? (double)scale_of_code<KIND>(scode) * (double)st : 0.0;
    const double sv = neg ? -(double)mag : (double)mag;
    double sse = 0.0;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const uint32_t code = (w[j >> 3] >> (4 * (j & 7))) & 15u;
      const double v = code == 8u ? sv : ((code & 8u) ? -0.5 : 0.5) * (double)fp4_mag_x2(code & 7u);
      const double e = (double)xf[j] - v * sbst;
      sse = sse + e * e;
    }
    if (c == 0 || sse < best) {
      best = sse;
      bsel = (uint32_t)c;
      bcode = scode;
      bw0 = w[0];
      bw1 = w[1];
    }
  }
  cw = make_uint2(bw0, bw1);
  if (bcode == 0u)
    sbyte = 0u;  // zero block: no metadata
  else
    sbyte = (KIND == kWeight) ? (((bsel & 1u) << 7) | ((bsel >> 1) << 6) | bcode) : ((bsel << 7) | bcode);
}

// Block values from the 16 input elements' bytes (fp32: 4 x 16 B, 16-bit: 2 x 16 B).
template <typename T> __device__ __forceinline__ void unpack_block(const u32x4_t* q, float (&v)[16]);
template <> __device__ __forceinline__ void unpack_block<float>(const u32x4_t* q, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) v[4 * i + j] = u2f(q[i][j]);
}
template <> __device__ __forceinline__ void unpack_block<__bf16>(const u32x4_t* q, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      v[8 * i + 2 * j] = u2f(q[i][j] << 16);
      v[8 * i + 2 * j + 1] = u2f(q[i][j] & 0xFFFF0000u);
    }
}
template <> __device__ __forceinline__ void unpack_block<_Float16>(const u32x4_t* q, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      v[8 * i + 2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(q[i][j] & 0xFFFFu));
      v[8 * i + 2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(q[i][j] >> 16));
    }
}

// Each wave takes 64 consecutive blocks per step: its 16-byte loads cover the
// blocks' bytes contiguously (1 KiB per instruction; a block per lane would
// spread every instruction over 2-4 KiB), go to a per-wave LDS stage and come
// back as one block per lane.  The next step's loads are in flight while a
// step is encoded; the buffer descriptor is rebased per step, so a read past
// the tensor returns zero and any tensor size works with 32-bit offsets.
// Encode-kernel modes: RaZeR (with the plain-NVFP4 no-remap option), the Four
// Over Six baseline, RaZeR with rescaled large special values.
enum { kModeRazer = 0, kModeFos = 1, kModeRescale = 2 };

template <int KIND, typename T, int MODE>
__global__ __launch_bounds__(256) void encode_kernel(const T* __restrict__ x, int64_t nblk,
                                                     const uint32_t* __restrict__ partial,
                                                     int npartial, uint2* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     float* __restrict__ ts_out, EncodeParams prm) {
  constexpr float kSMax = KIND == kWeight ? 30.0f : 448.0f;
  constexpr int kBB = 16 * (int)sizeof(T);  // input bytes per block
  constexpr int kNI = kBB * 64 / 1024;      // 16-byte loads per lane and step
  __shared__ __attribute__((aligned(16))) uint8_t stage[4][64 * kBB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t step = (int64_t)gridDim.x * 4 * 64;  // blocks per grid step
  int64_t bb = ((int64_t)blockIdx.x * 4 + wave) * 64;
  const uint8_t* xb = (const uint8_t*)x;
  const int64_t total = nblk * kBB;
  auto load = [&](int64_t b0, u32x4_t (&v)[kNI]) {
    const int64_t rem = total - b0 * kBB;
    const int nrec = rem <= 0 ? 0 : (int)min(rem, (int64_t)64 * kBB);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(xb + (rem <= 0 ? 0 : b0 * kBB)), (short)0, nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < kNI; i++) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (i * 64 + lane) * 16, 0, 2);
  };
  // The first step's blocks do not depend on the tensor amax: their loads are
  // in flight while the partials are folded.
  u32x4_t cur[kNI], nxt[kNI];
  load(bb, cur);

  uint32_t m = 0u;
  for (int i = threadIdx.x; i < npartial; i += 256) m = max(m, partial[i]);
  m = wave_max_u32(m);
  __shared__ uint32_t sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  m = max(max(sm[0], sm[1]), max(sm[2], sm[3]));
  const bool nonfinite = m >= 0x7F800000u;
  const float amax = u2f(m);
  const float st = amax / (6.0f * kSMax);
  if (blockIdx.x == 0 && threadIdx.x == 0) *ts_out = nonfinite ? __builtin_nanf("") : st;
  const bool all_zero = nonfinite || amax == 0.0f;
  const float rinv = 1.0f / amax;
  __shared__ float rtab[kScaleCodes<KIND>];
  if constexpr (MODE != kModeFos) {
    build_rcp_table<KIND>(rtab, st);
    __syncthreads();
  }

  if (all_zero) {
    for (; bb < nblk; bb += step)
      if (bb + lane < nblk) {
        codes[bb + lane] = make_uint2(0u, 0u);
        scales[bb + lane] = 0;
      }
    return;
  }
  // Drain the first loads here: otherwise the loop head, which the compiler
  // enters from two paths, waits (for the later steps) on the previous step's
  // stores as well.
#pragma unroll
  for (int i = 0; i < kNI; i++) asm volatile("" ::"v"(cur[i]));
  auto run = [&](auto fastdiv) {
    constexpr bool kFastDiv = decltype(fastdiv)::value;
    uint8_t* stg = stage[wave];
    for (; bb < nblk; bb += step) {
      load(bb + step, nxt);
#pragma unroll
      for (int i = 0; i < kNI; i++) *(u32x4_t*)(stg + (i * 64 + lane) * 16) = cur[i];
      wave_lds_sync();
      u32x4_t q[kBB / 16];
#pragma unroll
      for (int i = 0; i < kBB / 16; i++) q[i] = *(const u32x4_t*)(stg + lane * kBB + 16 * i);
      wave_lds_sync();
      float xf[16];
      unpack_block<T>(q, xf);
      uint2 cw;
      uint32_t sbyte;
      if constexpr (MODE == kModeFos)
        encode_block_fos<KIND>(xf, amax, st, cw, sbyte);
      else if constexpr (MODE == kModeRescale)
        encode_block_rescale<KIND>(xf, amax, st, rtab, prm, cw, sbyte);
      else
        encode_block<KIND, kFastDiv>(xf, amax, rinv, rtab, prm, cw, sbyte);
      // Buffer stores sized to the wave's valid blocks: lanes past the end are
      // dropped by the range check, so the stores need no branch (a branch
      // around them made every step wait for its stores to complete).
      const int nval = (int)min(nblk - bb, (int64_t)64);
      __builtin_amdgcn_raw_buffer_store_b64(
          u32x2_t{cw.x, cw.y}, __builtin_amdgcn_make_buffer_rsrc((void*)(codes + bb), (short)0, nval * 8, 0x00020000),
          lane * 8, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b8(
          (uint8_t)sbyte, __builtin_amdgcn_make_buffer_rsrc((void*)(scales + bb), (short)0, nval, 0x00020000), lane,
          0, 0);
#pragma unroll
      for (int i = 0; i < kNI; i++) cur[i] = nxt[i];
    }
  };
  // The Markstein quotient is used for 16-bit inputs whose amax keeps every
  // operand normal; the test is uniform, so the kernel takes one loop or the other.
  if constexpr (sizeof(T) == 2 && MODE == kModeRazer) {
    if (amax >= 0x1p-60f && amax <= 0x1p60f)
      run(std::true_type{});
    else
      run(std::false_type{});
  } else {
    run(std::false_type{});
  }
}

template <int KIND, typename T>
static hipError_t run_quantize(const T* x, const PackedView& out, uint32_t* partial,
                               hipStream_t stream) {
  const int64_t n = out.rows * out.cols;
  const int64_t nblk = n / 16;
  const int64_t nvec = n / (16 / (int64_t)sizeof(T));
  const int64_t g1 = amax_grid(nvec);
  launch_amax_partial<T>(dim3((unsigned)g1), stream,
                     (const uint4*)x, nvec, partial);
  EncodeParams prm;
  const int npairs = KIND == kWeight ? 2 : 1;
  for (int p = 0; p < 2; p++) {
    Candidate c = make_candidate(out.off_half[p < npairs ? p : 0]);
    prm.lo[p] = c.lo;
    prm.hi[p] = c.hi;
    prm.mag_x2[p] = c.mag_x2;
    prm.f[p] = make_pair_fast(out.off_half[p < npairs ? p : 0]);
  }
  prm.remap = (out.flags & kFlagNoRemap) ? 0 : 1;
  if (KIND == kAct && prm.f[0].hi > prm.f[0].lo && std::isfinite(prm.f[0].hi)) {
    const float m = 6.0f + 0.5f * (float)out.off_half[0];
    if (m - prm.lo[0] == prm.hi[0] - m) {  // M midway between its FP4 neighbours
      prm.sym = 1;
      prm.sym_m = m;
      prm.sym_h = 2.0f * (m - prm.lo[0]);
    }
  }
  int64_t g2 = (nblk + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (g2 > cap) g2 = cap;
  if (g2 < 1) g2 = 1;
  // Four Over Six takes precedence over the others, no-remap over the rescale
  if (out.flags & kFlagFourOverSix)
    hipLaunchKernelGGL((encode_kernel<KIND, T, kModeFos>), dim3((unsigned)g2), dim3(256), 0, stream, x,
                       nblk, partial, (int)g1, (uint2*)out.codes, out.scales, out.tensor_scale, prm);
  else if ((out.flags & kFlagRescale) && prm.remap)
    hipLaunchKernelGGL((encode_kernel<KIND, T, kModeRescale>), dim3((unsigned)g2), dim3(256), 0, stream, x,
                       nblk, partial, (int)g1, (uint2*)out.codes, out.scales, out.tensor_scale, prm);
  else
    hipLaunchKernelGGL((encode_kernel<KIND, T, kModeRazer>), dim3((unsigned)g2), dim3(256), 0, stream, x,
                       nblk, partial, (int)g1, (uint2*)out.codes, out.scales, out.tensor_scale, prm);
  return hipGetLastError();
}

// ---- second-pair offset search (offline weight encoder) -------------------------
// "RaZeR ..." (papernotes.org notes), Loss function / training strategy: the
// extra weight pair is chosen offline by a grid search.  For every offset o in
// -7..7 of the second pair, the tensor is encoded exactly as
// razer_quantize_weight does with offsets (off0, o) -- encode_block below is
// the same function -- and the squared reconstruction error
// (x - value * sb * st)^2 is summed in fp64 (value * sb * st is exact in fp64).
constexpr int kNumOffsets = 15;

struct OffsetSearchParams {
  EncodeParams base;  // pair 0 as given; pair 1 replaced per offset
  float lo1[kNumOffsets], hi1[kNumOffsets];
  int mag1[kNumOffsets];
  PairFast f1[kNumOffsets];
  float m0;           // |SV| of pair 0
};

template <typename T>
__global__ __launch_bounds__(256) void offset_sse_kernel(const T* __restrict__ x, int64_t nblk,
                                                         const uint32_t* __restrict__ partial,
                                                         int npartial, OffsetSearchParams prm,
                                                         double* __restrict__ part_out) {
  constexpr int kBB = 16 * (int)sizeof(T);
  constexpr int kNI = kBB * 64 / 1024;
  __shared__ __attribute__((aligned(16))) uint8_t stage[4][64 * kBB];
  __shared__ double acc[kNumOffsets][256];
  uint32_t m = 0u;
  for (int i = threadIdx.x; i < npartial; i += 256) m = max(m, partial[i]);
  m = wave_max_u32(m);
  __shared__ uint32_t sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  for (int o = 0; o < kNumOffsets; o++) acc[o][threadIdx.x] = 0.0;
  __syncthreads();
  m = max(max(sm[0], sm[1]), max(sm[2], sm[3]));
  const bool nonfinite = m >= 0x7F800000u;
  const float amax = u2f(m);
  const float st = amax / (6.0f * 30.0f);
  __shared__ float rtab[kScaleCodes<kWeight>];
  build_rcp_table<kWeight>(rtab, st);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t step = (int64_t)gridDim.x * 4 * 64;
  int64_t bb = ((int64_t)blockIdx.x * 4 + wave) * 64;
  if (!nonfinite && amax != 0.0f) {
    const uint8_t* xb = (const uint8_t*)x;
    const int64_t total = nblk * kBB;
    auto load = [&](int64_t b0, u32x4_t (&v)[kNI]) {
      const int64_t rem = total - b0 * kBB;
      const int nrec = rem <= 0 ? 0 : (int)min(rem, (int64_t)64 * kBB);
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc((void*)(xb + (rem <= 0 ? 0 : b0 * kBB)), (short)0, nrec, 0x00020000);
#pragma unroll
      for (int i = 0; i < kNI; i++) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (i * 64 + lane) * 16, 0, 2);
    };
    const double st64 = (double)st;
    u32x4_t cur[kNI], nxt[kNI];
    load(bb, cur);
    uint8_t* stg = stage[wave];
    for (; bb < nblk; bb += step) {
      load(bb + step, nxt);
#pragma unroll
      for (int i = 0; i < kNI; i++) *(u32x4_t*)(stg + (i * 64 + lane) * 16) = cur[i];
      wave_lds_sync();
      u32x4_t q[kBB / 16];
#pragma unroll
      for (int i = 0; i < kBB / 16; i++) q[i] = *(const u32x4_t*)(stg + lane * kBB + 16 * i);
      wave_lds_sync();
      float xf[16];
      unpack_block<T>(q, xf);
      if (bb + lane < nblk) {
#pragma unroll 1
        for (int o = 0; o < kNumOffsets; o++) {
          EncodeParams e = prm.base;
          e.lo[1] = prm.lo1[o];
          e.hi[1] = prm.hi1[o];
          e.mag_x2[1] = prm.mag1[o];
          e.f[1] = prm.f1[o];
          uint2 cw;
          uint32_t sbyte;
          encode_block<kWeight>(xf, amax, 0.0f, rtab, e, cw, sbyte);
          const double sbst = (double)scale_of_byte<kWeight>(sbyte) * st64;
          // the special value's sign is bit 7 of the scale byte, not the code's
          const double svm = (double)((sbyte & 0x40u) ? 0.5f * (float)prm.mag1[o] : prm.m0);
          const double sv = (sbyte & 0x80u) ? -svm : svm;
          double err = 0.0;
#pragma unroll
          for (int j = 0; j < 16; j++) {
            const uint32_t c = ((j < 8 ? cw.x : cw.y) >> (4 * (j & 7))) & 15u;
            const double mag = 0.5 * (double)fp4_mag_x2(c & 7u);
            const double v = ((c == 8u) ? sv : ((c & 8u) ? -mag : mag)) * sbst;
            const double d = (double)xf[j] - v;
            err += d * d;
          }
          acc[o][threadIdx.x] += err;
        }
      }
#pragma unroll
      for (int i = 0; i < kNI; i++) cur[i] = nxt[i];
    }
  }
  __syncthreads();
  if (threadIdx.x < kNumOffsets) {
    double sum = 0.0;
    for (int t = 0; t < 256; t++) sum += acc[threadIdx.x][t];
    part_out[(int64_t)blockIdx.x * kNumOffsets + threadIdx.x] = nonfinite ? __builtin_nan("") : sum;
  }
}

// One workgroup per offset: strided partial sums, then a fixed-shape LDS tree,
// so the result does not depend on timing.
__global__ __launch_bounds__(256) void offset_sse_reduce_kernel(const double* __restrict__ part, int nwg,
                                                                double* __restrict__ sse) {
  __shared__ double red[256];
  const int o = blockIdx.x;
  double sum = 0.0;
  for (int g = threadIdx.x; g < nwg; g += 256) sum += part[(int64_t)g * kNumOffsets + o];
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) sse[o] = red[0];
}

static int64_t offset_search_grid(int64_t nblk) {
  int64_t g = (nblk + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 4;
  if (g > cap) g = cap;
  return g < 1 ? 1 : g;
}

size_t offset_search_ws_bytes(int64_t n) {
  return kAmaxMaxPartials * sizeof(uint32_t) +
         (size_t)offset_search_grid(n / 16) * kNumOffsets * sizeof(double);
}

template <typename T>
static hipError_t run_offset_search(const T* x, int64_t n, int off0, double* sse, void* ws,
                                    hipStream_t stream) {
  const int64_t nblk = n / 16;
  uint32_t* partial = (uint32_t*)ws;
  double* part = (double*)((uint8_t*)ws + kAmaxMaxPartials * sizeof(uint32_t));
  const int64_t nvec = n / (16 / (int64_t)sizeof(T));
  const int64_t g1 = amax_grid(nvec);
  if (nvec > 0)
    launch_amax_partial<T>(dim3((unsigned)g1), stream,
                       (const uint4*)x, nvec, partial);
  OffsetSearchParams prm;
  for (int p = 0; p < 2; p++) {
    const Candidate c = make_candidate(off0);
    prm.base.lo[p] = c.lo;
    prm.base.hi[p] = c.hi;
    prm.base.mag_x2[p] = c.mag_x2;
    prm.base.f[p] = make_pair_fast(off0);
  }
  prm.base.remap = 1;
  prm.m0 = 6.0f + 0.5f * (float)off0;
  for (int o = 0; o < kNumOffsets; o++) {
    const Candidate c = make_candidate(o - 7);
    prm.lo1[o] = c.lo;
    prm.hi1[o] = c.hi;
    prm.mag1[o] = c.mag_x2;
    prm.f1[o] = make_pair_fast(o - 7);
  }
  const int64_t g2 = offset_search_grid(nblk);
  if (nvec > 0) {
    hipLaunchKernelGGL(offset_sse_kernel<T>, dim3((unsigned)g2), dim3(256), 0, stream, x, nblk, partial,
                       (int)g1, prm, part);
  } else {
    hipLaunchKernelGGL(offset_sse_reduce_kernel, dim3(kNumOffsets), dim3(256), 0, stream, (const double*)nullptr, 0, sse);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(offset_sse_reduce_kernel, dim3(kNumOffsets), dim3(256), 0, stream, (const double*)part, (int)g2, sse);
  return hipGetLastError();
}

hipError_t launch_offset_search(const void* x, int dtype, int64_t rows, int64_t cols, int off0,
                                double* sse, void* ws, hipStream_t stream) {
  const int64_t n = rows * cols;
  if (dtype == kF32) return run_offset_search((const float*)x, n, off0, sse, ws, stream);
  if (dtype == kF16) return run_offset_search((const _Float16*)x, n, off0, sse, ws, stream);
  return run_offset_search((const __bf16*)x, n, off0, sse, ws, stream);
}

// ---- block-size and scale-format variants ------------------------------------
// "RaZeR ..." notes, Key findings (blocks of 32, 64 and 128 elements) and Key
// design 3 (FP16 block scales for 128-element groups with the metadata in the
// scale's sign bit and top exponent bit).  The same steps as encode_block for
// a block of 16 << glog2 elements: each lane still holds 16 consecutive
// elements, and the 2^glog2 lanes of a block (adjacent lanes of one wave)
// combine their block maximum, their candidate error changes and, for Four
// Over Six, their squared errors.  Candidate changes are summed in fp64,
// where every change (v - q)(v + q - 2y) and every sum of them is exact (a
// moved element has |y| > 2, so each term is a multiple of 2^-23 below 2^5),
// so the comparison does not depend on the order of the sums.  Four Over Six
// errors are not exact, so they are added in element order: the running sum
// passes from lane to lane of the block (block_sse_in_order).
struct VariantParams {
  double cand[4];  // +M0, -M0 (, +M1, -M1), in selection-index order
  int ncand;
  int glog2;       // lanes per block = 2^glog2
  int sfmt;        // 0 byte scales, 1 FP16 group scales
  int mode;        // 0 plain NVFP4, 1 RaZeR, 2 Four Over Six
};

__device__ __forceinline__ float group_max(float v, int glog2) {
  for (int m = 1; m < (1 << glog2); m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// exact fp64 sums only: the butterfly adds in a lane-dependent order
__device__ __forceinline__ double group_sum_exact(double v, int glog2) {
  for (int m = 1; m < (1 << glog2); m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Squared error of a plain-FP4 block spread over 2^glog2 adjacent lanes (16
// elements each), summed in element order: lane i of the block continues the
// running sum of lanes 0 .. i-1 over its own 16 elements.  Every lane computes
// its continuation of the current sum and the block takes lane i's.
__device__ __forceinline__ double block_sse_in_order(const float (&xf)[16], const uint32_t (&w)[2],
                                                     float sb, float st, int glog2, int lane) {
  const int g0 = lane & ~((1 << glog2) - 1);
  double s = 0.0;
  for (int i = 0; i < (1 << glog2); i++) s = __shfl(plain_block_sse(xf, w, sb, st, s), g0 + i);
  return s;
}

// One plain-FP4 encoding of the lane's 16 elements at real block scale sb_real:
// scale code (0: zero block, then sb = 0 and all codes +0), the decoded scale,
// the scaled values and the codes.
template <int KIND>
__device__ __forceinline__ uint32_t variant_at_scale(const float (&xf)[16], float sb_real, float st,
                                                     int sfmt, uint32_t (&w)[2], float (&y)[16],
                                                     float& sb) {
  w[0] = 0u;
  w[1] = 0u;
#pragma unroll
  for (int j = 0; j < 16; j++) y[j] = 0.0f;
  uint32_t scode = sfmt ? min((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)sb_real), 0x3FFFu)
                        : round_scale<KIND>(sb_real);
  sb = 0.0f;
  if (scode == 0u) return 0u;
  sb = sfmt ? scale_of_f16word(scode) : scale_of_code<KIND>(scode);
  const float d = sb * st;
  const float rcp = 1.0f / d;
  if (!(rcp < INFINITY)) {
    sb = 0.0f;
    return 0u;
  }
#pragma unroll
  for (int j = 0; j < 16; j++) y[j] = xf[j] * rcp;
  fp4_pack16(y, w);
  return scode;
}

template <int KIND>
__device__ __forceinline__ void encode_variant(const float (&xf)[16], float amax, float st,
                                               const VariantParams& vp, int lane, uint2& cw,
                                               uint32_t& sword) {
#pragma clang fp contract(off)
  const float smax = vp.sfmt ? kF16ScaleMax : (KIND == kWeight ? 30.0f : 448.0f);
  float amax_b = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; j++) amax_b = fmaxf(amax_b, fabsf(xf[j]));
  amax_b = group_max(amax_b, vp.glog2);
  const float r = amax_b / amax;
  const float sb_real = r * smax;
  uint32_t w[2];
  float y[16], sb;
  uint32_t scode = variant_at_scale<KIND>(xf, sb_real, st, vp.sfmt, w, y, sb);
  uint32_t sel = 0u;
  if (vp.mode == 2) {
    uint32_t w4[2];
    float y4[16], sb4;
    const uint32_t c4 = variant_at_scale<KIND>(xf, sb_real * 1.5f, st, vp.sfmt, w4, y4, sb4);
    const double e6 = block_sse_in_order(xf, w, sb, st, vp.glog2, lane);
    const double e4 = block_sse_in_order(xf, w4, sb4, st, vp.glog2, lane);
    if (e4 < e6) {
      w[0] = w4[0];
      w[1] = w4[1];
      scode = c4;
    }
  } else if (vp.mode == 1 && scode != 0u) {  // scode is the same on every lane of the block
    double q0[16];
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const uint32_t c = (w[j >> 3] >> (4 * (j & 7))) & 15u;
      const double m = 0.5 * (double)fp4_mag_x2(c & 7u);
      q0[j] = (c & 8u) ? -m : m;
    }
    double delta[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int c = 0; c < 4; c++) {
      if (c < vp.ncand) {
        const double v = vp.cand[c];
        double acc = 0.0;
#pragma unroll
        for (int j = 0; j < 16; j++) {
          const double yj = (double)y[j];
          if (fabs(yj - v) < fabs(yj - q0[j])) acc += (v - q0[j]) * (v + q0[j] - 2.0 * yj);
        }
        delta[c] = group_sum_exact(acc, vp.glog2);
      }
    }
    double best = delta[0];
#pragma unroll
    for (int c = 1; c < 4; c++)
      if (c < vp.ncand && delta[c] < best) {
        best = delta[c];
        sel = (uint32_t)c;
      }
    const double v = sel == 0u ? vp.cand[0] : sel == 1u ? vp.cand[1] : sel == 2u ? vp.cand[2] : vp.cand[3];
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const double yj = (double)y[j];
      const uint32_t sh = 4 * (j & 7);
      if (fabs(yj - v) < fabs(yj - q0[j])) w[j >> 3] = (w[j >> 3] & ~(15u << sh)) | (8u << sh);
    }
  }
  cw = make_uint2(w[0], w[1]);
  if (scode == 0u) sel = 0u;
  if (vp.sfmt)
    sword = ((sel & 1u) << 15) | ((sel >> 1) << 14) | scode;
  else
    sword = KIND == kWeight ? (((sel & 1u) << 7) | ((sel >> 1) << 6) | scode) : ((sel << 7) | scode);
}

// Same staging as encode_kernel (64 consecutive 16-element runs per wave and
// step); the first lane of each block writes its scale (1 or 2 bytes).
template <int KIND, typename T>
__global__ __launch_bounds__(256) void encode_variant_kernel(const T* __restrict__ x, int64_t nsub,
                                                             const uint32_t* __restrict__ partial,
                                                             int npartial, uint2* __restrict__ codes,
                                                             uint8_t* __restrict__ scales,
                                                             float* __restrict__ ts_out, VariantParams vp) {
  constexpr int kBB = 16 * (int)sizeof(T);
  constexpr int kNI = kBB * 64 / 1024;
  __shared__ __attribute__((aligned(16))) uint8_t stage[4][64 * kBB];
  uint32_t m = 0u;
  for (int i = threadIdx.x; i < npartial; i += 256) m = max(m, partial[i]);
  m = wave_max_u32(m);
  __shared__ uint32_t sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  m = max(max(sm[0], sm[1]), max(sm[2], sm[3]));
  const bool nonfinite = m >= 0x7F800000u;
  const float amax = u2f(m);
  const float smax = vp.sfmt ? kF16ScaleMax : (KIND == kWeight ? 30.0f : 448.0f);
  const float st = amax / (6.0f * smax);
  if (blockIdx.x == 0 && threadIdx.x == 0) *ts_out = nonfinite ? __builtin_nanf("") : st;
  const bool all_zero = nonfinite || amax == 0.0f;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool leader = (lane & ((1 << vp.glog2) - 1)) == 0;
  const int64_t step = (int64_t)gridDim.x * 4 * 64;
  int64_t bb = ((int64_t)blockIdx.x * 4 + wave) * 64;
  auto store = [&](int64_t sub, uint2 cw, uint32_t sword) {
    if (sub >= nsub) return;
    codes[sub] = cw;
    if (leader) {
      const int64_t blk = sub >> vp.glog2;
      if (vp.sfmt) ((uint16_t*)scales)[blk] = (uint16_t)sword;
      else scales[blk] = (uint8_t)sword;
    }
  };
  if (all_zero) {
    for (; bb < nsub; bb += step) store(bb + lane, make_uint2(0u, 0u), 0u);
    return;
  }
  const uint8_t* xb = (const uint8_t*)x;
  const int64_t total = nsub * kBB;
  auto load = [&](int64_t b0, u32x4_t (&v)[kNI]) {
    const int64_t rem = total - b0 * kBB;
    const int nrec = rem <= 0 ? 0 : (int)min(rem, (int64_t)64 * kBB);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(xb + (rem <= 0 ? 0 : b0 * kBB)), (short)0, nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < kNI; i++) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (i * 64 + lane) * 16, 0, 2);
  };
  u32x4_t cur[kNI], nxt[kNI];
  load(bb, cur);
  uint8_t* stg = stage[wave];
  for (; bb < nsub; bb += step) {
    load(bb + step, nxt);
#pragma unroll
    for (int i = 0; i < kNI; i++) *(u32x4_t*)(stg + (i * 64 + lane) * 16) = cur[i];
    wave_lds_sync();
    u32x4_t q[kBB / 16];
#pragma unroll
    for (int i = 0; i < kBB / 16; i++) q[i] = *(const u32x4_t*)(stg + lane * kBB + 16 * i);
    wave_lds_sync();
    float xf[16];
    unpack_block<T>(q, xf);
    uint2 cw;
    uint32_t sword;
    encode_variant<KIND>(xf, amax, st, vp, lane, cw, sword);
    store(bb + lane, cw, sword);
#pragma unroll
    for (int i = 0; i < kNI; i++) cur[i] = nxt[i];
  }
}

template <int KIND, typename T>
static hipError_t run_quantize_variant(const T* x, const PackedView& out, uint32_t* partial,
                                       hipStream_t stream) {
  const int64_t n = out.rows * out.cols;
  const int64_t nsub = n / 16;
  const int64_t nvec = n / (16 / (int64_t)sizeof(T));
  const int64_t g1 = amax_grid(nvec);
  launch_amax_partial<T>(dim3((unsigned)g1), stream,
                     (const uint4*)x, nvec, partial);
  VariantParams vp;
  const int npairs = KIND == kWeight ? 2 : 1;
  for (int p = 0; p < npairs; p++) {
    const double M = 6.0 + 0.5 * out.off_half[p];
    vp.cand[2 * p] = M;
    vp.cand[2 * p + 1] = -M;
  }
  for (int c = 2 * npairs; c < 4; c++) vp.cand[c] = 0.0;
  vp.ncand = 2 * npairs;
  vp.glog2 = out.blog2 - 4;
  vp.sfmt = out.sfmt;
  vp.mode = (out.flags & kFlagFourOverSix) ? 2 : (out.flags & kFlagNoRemap) ? 0 : 1;
  int64_t g2 = (nsub + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (g2 > cap) g2 = cap;
  if (g2 < 1) g2 = 1;
  hipLaunchKernelGGL((encode_variant_kernel<KIND, T>), dim3((unsigned)g2), dim3(256), 0, stream, x,
                     nsub, partial, (int)g1, (uint2*)out.codes, out.scales, out.tensor_scale, vp);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int dtype, const PackedView& out, void* ws,
                           hipStream_t stream) {
  uint32_t* partial = (uint32_t*)ws;
  if (!default_layout(out)) {
    if (out.kind == kWeight) {
      if (dtype == kF32) return run_quantize_variant<kWeight>((const float*)x, out, partial, stream);
      if (dtype == kF16) return run_quantize_variant<kWeight>((const _Float16*)x, out, partial, stream);
      return run_quantize_variant<kWeight>((const __bf16*)x, out, partial, stream);
    }
    if (dtype == kF32) return run_quantize_variant<kAct>((const float*)x, out, partial, stream);
    if (dtype == kF16) return run_quantize_variant<kAct>((const _Float16*)x, out, partial, stream);
    return run_quantize_variant<kAct>((const __bf16*)x, out, partial, stream);
  }
  if (out.kind == kWeight) {
    if (dtype == kF32) return run_quantize<kWeight>((const float*)x, out, partial, stream);
    if (dtype == kF16) return run_quantize<kWeight>((const _Float16*)x, out, partial, stream);
    return run_quantize<kWeight>((const __bf16*)x, out, partial, stream);
  }
  if (dtype == kF32) return run_quantize<kAct>((const float*)x, out, partial, stream);
  if (dtype == kF16) return run_quantize<kAct>((const _Float16*)x, out, partial, stream);
  return run_quantize<kAct>((const __bf16*)x, out, partial, stream);
}

// ---- allocation-free activation encoder ---------------------------------------
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops): the amax partials live in a file-scope device array instead
// of a caller workspace.  Each device holds its own copy for the life of the
// process; host code uses the address hipGetSymbolAddress returns for the
// current device (the array's name is only a host-side stand-in).  Every call
// on one device shares that copy, so calls that overlap on one device race.
// Pass 1 writes every partial that pass 2 reads, so nothing needs clearing.
constexpr size_t kNoAllocScratchBytes = 4096;
static_assert(kAmaxMaxPartials * sizeof(uint32_t) <= kNoAllocScratchBytes,
              "the encoder's partials must fit the static scratch");

}  // namespace rz

static __device__ __align__(256) uint8_t scratch[rz::kNoAllocScratchBytes];

namespace rz {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

// The current device's copy of the scratch array, resolved once per device.
hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_quantize_noalloc(const void* x, int dtype, const PackedView& out, hipStream_t stream) {
  if (quantize_ws_bytes() > kNoAllocScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_quantize(x, dtype, out, ws, stream);
}

}  // namespace rz
