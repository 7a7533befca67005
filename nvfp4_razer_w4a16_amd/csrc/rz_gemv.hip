// rz_gemv.hip -- batch-1 W4A16 product y = x * W^T on gfx950, decoding the
// RaZeR weight format in registers.
//
// "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
// Remapping" (papernotes.org notes), Key design 3: weight-only GEMV kernels
// decode the packed weights inside the kernel, and the launch is sized so
// small matrices are not over-split; "Technical Summary: RaZeR ..."
// (gist.science), §2.3.  The pages' kernel (group-128 FP16 scales on another
// GPU) is prior art only; this one is written for CDNA4:
//   - streaming: a wavefront keeps its slice of x in registers for the whole
//     launch and walks a run of weight rows, with the code loads of the next D
//     rows in flight while it decodes the current one, so the decode work of
//     every wave overlaps the HBM stream instead of waiting behind it;
//   - lane l of a wave takes chunks (32 or 16 elements) l, l+64, ... of the
//     wave's K slice, so every 16-byte code load is one coalesced 1 KiB wave
//     access; for long rows the K range is split over KS waves of a workgroup
//     and their row sums are added in LDS;
//   - the scale bytes of a row quad arrive with one 8- or 4-byte load per lane
//     (issued before the codes) and reach their lanes through a per-wave LDS
//     stage, instead of a 1- or 2-byte load per lane and row;
//   - codes become fp16/bf16 pairs with the gfx950 packed FP4 conversion and
//     are contracted with x by v_dot2 (fp32 accumulate).  The remapped code
//     0b1000 converts to -0 (0x8000), the smallest pair half when read as
//     int16; a packed int16 max against -0.25 replaces exactly those halves by
//     -0.25 (every other converted value is +0 or has magnitude >= 0.5).  With
//     d0 = x . q and d1 = x . max(q, -0.25) the block sum is
//     d0 + SV * S = d0 * (1 + 4 SV) - 4 SV * d1, where S sums x over the
//     remapped positions; a 256-entry LDS table holds the two coefficients
//     (times the block scale) for every scale byte;
//   - each row's 64 lane partials are summed with DPP and scaled once by the
//     tensor scale.
#include "rz_device.h"
#include "rz_launch.h"

#include <type_traits>

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

// The converted pair with remapped halves (-0) replaced by -0.25.
template <typename XT>
__device__ __forceinline__ typename Pair<XT>::T mark_remapped(typename Pair<XT>::T p) {
  const short2_t q = __builtin_elementwise_max(__builtin_bit_cast(short2_t, p),
                                               (short2_t){Pair<XT>::kQuarterNeg, Pair<XT>::kQuarterNeg});
  return __builtin_bit_cast(typename Pair<XT>::T, q);
}

// One 16-element block (codes w0: elements 0..7, w1: 8..15; byte j of a word
// holds elements 2j, 2j+1, low nibble first) against 8 x pairs: d0 = x . q and
// d1 = x . max(q, -0.25).  All conversions come first so that no dot reads a
// register written by the instruction just before it.
template <typename XT>
__device__ __forceinline__ void block_dot(uint32_t w0, uint32_t w1, const typename Pair<XT>::T* xp,
                                          float& d0, float& d1) {
  typedef typename Pair<XT>::T P;
  P p[8], m[8];
  p[0] = Pair<XT>::template cvt<0>(w0);
  p[1] = Pair<XT>::template cvt<1>(w0);
  p[2] = Pair<XT>::template cvt<2>(w0);
  p[3] = Pair<XT>::template cvt<3>(w0);
  p[4] = Pair<XT>::template cvt<0>(w1);
  p[5] = Pair<XT>::template cvt<1>(w1);
  p[6] = Pair<XT>::template cvt<2>(w1);
  p[7] = Pair<XT>::template cvt<3>(w1);
#pragma unroll
  for (int j = 0; j < 8; j++) m[j] = mark_remapped<XT>(p[j]);
  d0 = 0.0f;
  d1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    d0 = Pair<XT>::dot(p[j], xp[j], d0);
    d1 = Pair<XT>::dot(m[j], xp[j], d1);
  }
}

// Lane sums of four values at once.  v_permlane32_swap exchanges lanes 32..63
// of its first operand with lanes 0..31 of its second, v_permlane16_swap the
// odd 16-lane rows of the first with the even rows of the second (gfx950), so
// two swap+add steps leave, in 16-lane row rho, the sum over lanes l, l+16,
// l+32, l+48 of value {0, 2, 1, 3}[rho]; DPP then sums each row.  Every lane
// of row rho ends with the total of value quad_row(rho).
__device__ __forceinline__ float swap_sum32(float a, float b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}
__device__ __forceinline__ float swap_sum16(float a, float b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_sum(const float* a) {
  float v = swap_sum16(swap_sum32(a[0], a[1]), swap_sum32(a[2], a[3]));
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  return v;
}
__device__ __forceinline__ int quad_row(int lane) {
  const int rho = lane >> 4;
  return ((rho & 1) << 1) | (rho >> 1);
}

// One weight of a launch: its packed buffers, output, rows and decode
// parameters, and the first workgroup of the launch that works on it.
struct GemvWeight {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* ts;
  void* y;
  int64_t n;
  int kind;
  float m0, m1;
  int wg0;
};

// A launch covers up to kGemvGroupMax weights that share x and K (for example
// the gate and up projections of an MLP); workgroups [wg0(g), wg0(g+1)) work
// on weight g.
constexpr int kGemvGroupMax = 4;
struct GemvArgs {
  const void* x;
  GemvWeight w[kGemvGroupMax];
  int count;
  int64_t k, nchunk;
  int rpw;   // rows per workgroup
  int rpwv;  // rows per row group (multiple of 4)
  int ydt;
};

__device__ __forceinline__ void store_out(void* y, int64_t i, float v, int ydt) {
  if (ydt == kF32) ((float*)y)[i] = v;
  else if (ydt == kF16) ((_Float16*)y)[i] = (_Float16)v;
  else ((__bf16*)y)[i] = (__bf16)v;
}

// Raw buffer loads: a read past num_records returns zero and moves no data,
// which covers the ragged tail of K and the rows past the end of a run
// without branches around the loads.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;      // gfx950 raw buffer, 32-bit data format
constexpr int kOob = 0x40000000;             // past any num_records, also when added twice
constexpr int kNt = 2;                       // non-temporal: weights are read once

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, kRsrcWord3);
}

// Codes of one chunk (32 or 16 elements) of one row.
template <int UNIT> struct Chunk;
template <> struct Chunk<2> {  // 32 elements: 16 code bytes
  u32x4_t c;
  __device__ __forceinline__ void load(Rsrc cr, int coff) {
    c = __builtin_amdgcn_raw_buffer_load_b128(cr, coff, 0, kNt);
  }
  __device__ __forceinline__ uint32_t w(int j) const { return c[j]; }
};
template <> struct Chunk<1> {  // 16 elements: 8 code bytes
  u32x2_t c;
  __device__ __forceinline__ void load(Rsrc cr, int coff) {
    c = __builtin_amdgcn_raw_buffer_load_b64(cr, coff, 0, kNt);
  }
  __device__ __forceinline__ uint32_t w(int j) const { return c[j]; }
};

// Scale bytes of a row quad, 4 * UNIT per lane: lane l holds bytes
// 4 * UNIT * (l % 16) .. of row l / 16's segment (the 64 * UNIT bytes that
// cover one chunk index of all 64 lanes).  One wide load per lane replaces a
// 1- or 2-byte load per lane and row; the bytes reach their lanes through a
// per-wave LDS stage.
template <int UNIT, bool WIDE> struct ScaleWord;
template <> struct ScaleWord<2, true> {
  u32x2_t v;
  __device__ __forceinline__ void load(Rsrc sr, int off) { v = __builtin_amdgcn_raw_buffer_load_b64(sr, off, 0, 0); }
  __device__ __forceinline__ void store(uint8_t* p) const { *(u32x2_t*)p = v; }
};
template <> struct ScaleWord<1, true> {
  uint32_t v;
  __device__ __forceinline__ void load(Rsrc sr, int off) { v = __builtin_amdgcn_raw_buffer_load_b32(sr, off, 0, 0); }
  __device__ __forceinline__ void store(uint8_t* p) const { *(uint32_t*)p = v; }
};
// Scale rows whose stride breaks the wide loads' alignment: the same bytes
// with 2- or 1-byte loads.
template <> struct ScaleWord<2, false> {
  uint32_t h[4];
  __device__ __forceinline__ void load(Rsrc sr, int off) {
#pragma unroll
    for (int j = 0; j < 4; j++) h[j] = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 2 * j, 0);
  }
  __device__ __forceinline__ void store(uint8_t* p) const {
#pragma unroll
    for (int j = 0; j < 4; j++) *(uint16_t*)(p + 2 * j) = (uint16_t)h[j];
  }
};
template <> struct ScaleWord<1, false> {
  uint32_t b[4];
  __device__ __forceinline__ void load(Rsrc sr, int off) {
#pragma unroll
    for (int j = 0; j < 4; j++) b[j] = __builtin_amdgcn_raw_buffer_load_b8(sr, off, j, 0);
  }
  __device__ __forceinline__ void store(uint8_t* p) const {
#pragma unroll
    for (int j = 0; j < 4; j++) p[j] = (uint8_t)b[j];
  }
};

// FP16 group scales: one 2-byte word per lane and row quad (row lane / 16,
// block lane % 16 of the chunk index's 16 blocks), always aligned and inside
// the row.
struct ScaleHalf {
  uint32_t h;
  __device__ __forceinline__ void load(Rsrc sr, int off) { h = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0); }
  __device__ __forceinline__ void store(uint8_t* p) const { *(uint16_t*)p = (uint16_t)h; }
};

constexpr int kGemvMaxRpw = 64;  // rows per workgroup (bounds the LDS partials)

// Workgroup = 4 waves = KS K-slices x (4 / KS) row groups.  The workgroup's
// run of rows is walked in quads, dealt round-robin to the row groups (row
// group rg takes quads rg, rg + 4 / KS, ...: rpwv rows each), so at every quad
// step the workgroup reads one contiguous block of rows; within a row, wave
// (ks, rg) takes chunks (i * KS + ks) * 64 + lane for i < CPL.  The loads of the next
// NQ - 1 row quads are in flight while a quad is decoded.
//
// F16S: weights in the 128-element FP16-scale layout (UNIT 2).  A row quad's
// scales for one chunk index are 4 x 16 words; lane l loads word l % 16 of
// row l / 16, and a lane's chunk reads the word of its block (chunk / 4) from
// the stage.  Both 16-element halves of a chunk share that word, whose two
// coefficients come from the word itself.
template <typename XT, int UNIT, int CPL, int KS, int NQ, bool SW, bool F16S>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
  typedef typename Pair<XT>::T P;
  typedef typename std::conditional<F16S, ScaleHalf, ScaleWord<UNIT, SW>>::type SWord;
  constexpr int kPairs = 8 * UNIT;  // x pairs per chunk
  constexpr int kSeg = 64 * UNIT;  // scale bytes of one chunk index, one row
  __shared__ float2 lut[256];
  __shared__ float part[KS > 1 ? KS * kGemvMaxRpw : 1];
  __shared__ __attribute__((aligned(16))) uint8_t sstage[4][CPL][4][kSeg];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ks = wave % KS, rg = wave / KS;
  // this workgroup's weight (a uniform choice among at most four)
  GemvWeight w = a.w[0];
#pragma unroll
  for (int g = 1; g < kGemvGroupMax; g++)
    if (g < a.count && (int)blockIdx.x >= a.w[g].wg0) w = a.w[g];
  const int64_t base = (int64_t)((int)blockIdx.x - w.wg0) * a.rpw;
  const int rows_wg = (int)min((int64_t)a.rpw, w.n - base);
  // Quad q of row group rg covers rows 4 (q RW + rg) .. + 4 of the run, so the
  // row groups of a workgroup read one contiguous block of rows per quad step.
  constexpr int RW = 4 / KS;
  const int nquad = (rows_wg + 3) >> 2;
  const int nq = nquad > rg ? (nquad - rg + RW - 1) / RW : 0;  // quads of this wave
  const int rcb = (int)(a.k / 2), rsb = (int)(F16S ? a.k / 64 : a.k / 16);
  const Rsrc crs = make_rsrc(w.codes + base * rcb, (int64_t)rows_wg * rcb);
  const Rsrc srs = make_rsrc(w.scales + base * rsb, (int64_t)rows_wg * rsb);
  const Rsrc xrs = make_rsrc(a.x, a.k * 2);

  // Chunks of this wave: ni of them hold any valid lane (wave-uniform); a
  // lane past K reads nothing (offset kOob) and holds zero x.
  int ni = 0;
  int coff[CPL], sgo[CPL];
#pragma unroll
  for (int i = 0; i < CPL; i++) {
    const int c0 = (i * KS + ks) * 64;
    if (c0 < a.nchunk) ni = i + 1;
    const int c = c0 + lane;
    coff[i] = c < a.nchunk ? c * 8 * UNIT : kOob;
    // scale segment i, lane's 4 * UNIT bytes; past the row's end reads zero
    if (F16S) {
      const int sb0 = c0 / 2 + 2 * (lane & 15);
      sgo[i] = sb0 < rsb ? sb0 : kOob;
    } else {
      const int sb0 = (c0 + 4 * (lane & 15)) * UNIT;
      sgo[i] = c0 + 4 * (lane & 15) < a.nchunk ? sb0 : kOob;
    }
  }

  // x slice in registers, requested before any weight bytes.
  P xv[CPL][kPairs];
#pragma unroll
  for (int i = 0; i < CPL; i++) {
#pragma unroll
    for (int q = 0; q < kPairs / 4; q++) {
      const int off = coff[i] == kOob ? kOob : coff[i] * 4 + 16 * q;  // x: 4 bytes per code byte
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
      ((u32x4_t*)xv[i])[q] = v;
    }
  }

  Chunk<UNIT> buf[NQ][4][CPL];
  SWord sbuf[NQ][CPL];
  // scale bytes first: the table lookups wait on them, the dots on the codes
  auto load_quad = [&](int slot, int q) {
    const int srow = 4 * (q * RW + rg) + (lane >> 4);
    const int sbase = srow < rows_wg ? srow * rsb : kOob;
#pragma unroll
    for (int i = 0; i < CPL; i++) sbuf[slot][i].load(srs, sbase + sgo[i]);
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int crow = 4 * (q * RW + rg) + r;
      const int cb = crow < rows_wg ? crow * rcb : kOob;
#pragma unroll
      for (int i = 0; i < CPL; i++) buf[slot][r][i].load(crs, cb + coff[i]);
    }
  };
  // the first NQ quads are requested before the table is built
#pragma unroll
  for (int s = 0; s < NQ; s++) load_quad(s, s);

  {
    const uint32_t i = threadIdx.x;
    float sb, sv;
    if (w.kind == kWeight) {
      sb = scale_of_byte<kWeight>(i);
      sv = special_of_byte<kWeight>(i, w.m0, w.m1);
    } else {
      sb = scale_of_byte<kAct>(i);
      sv = special_of_byte<kAct>(i, w.m0, w.m1);
    }
    lut[i] = make_float2(sb * (1.0f + 4.0f * sv), -4.0f * sb * sv);
  }
  __syncthreads();
  const float st = *w.ts;
  const int my_row = quad_row(lane);  // the row of the quad this lane's sum belongs to
  uint8_t (*stg)[4][kSeg] = sstage[wave];

  for (int q0 = 0; q0 < nq; q0 += NQ) {
#pragma unroll
    for (int s = 0; s < NQ; s++) {
      const int q = q0 + s;
      if (q < nq) {
        // this quad's scale bytes to their lanes (one wave: no barrier)
#pragma unroll
        for (int i = 0; i < CPL; i++) {
          if (F16S) {
            sbuf[s][i].store(stg[i][lane >> 4] + 2 * (lane & 15));
          } else {
            sbuf[s][i].store(stg[i][lane >> 4] + 4 * UNIT * (lane & 15));
          }
        }
        wave_lds_sync();
        float acc[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
          acc[r] = 0.0f;
#pragma unroll
          for (int i = 0; i < CPL; i++) {
            if (F16S && i < ni) {
              const Chunk<UNIT>& ch = buf[s][r][i];
              const uint32_t sw = (uint32_t)*(const uint16_t*)(stg[i][r] + 2 * (lane >> 2));
              float d0a, d1a, d0b, d1b;
              block_dot<XT>(ch.w(0), ch.w(1), xv[i], d0a, d1a);
              block_dot<XT>(ch.w(2), ch.w(3), xv[i] + 8, d0b, d1b);
              const float sb = scale_of_f16word(sw), sv = special_of_f16word(sw, w.m0, w.m1);
              acc[r] = fmaf(d0a + d0b, sb * (1.0f + 4.0f * sv), acc[r]);
              acc[r] = fmaf(d1a + d1b, -4.0f * sb * sv, acc[r]);
            } else if (!F16S && i < ni) {
              const Chunk<UNIT>& ch = buf[s][r][i];
              const uint32_t sw = UNIT == 2 ? (uint32_t)*(const uint16_t*)(stg[i][r] + 2 * lane)
                                            : (uint32_t)stg[i][r][lane];
#pragma unroll
              for (int u = 0; u < UNIT; u++) {
                float d0, d1;
                block_dot<XT>(ch.w(2 * u), ch.w(2 * u + 1), xv[i] + 8 * u, d0, d1);
                const float2 f = lut[(sw >> (8 * u)) & 0xFFu];
                acc[r] = fmaf(d0, f.x, acc[r]);
                acc[r] = fmaf(d1, f.y, acc[r]);
              }
            }
          }
        }
        wave_lds_sync();       // stage reads done before the next quad's writes
        load_quad(s, q + NQ);  // refill the slot
        const float v = quad_sum(acc);
        const int orow = 4 * (q * RW + rg) + my_row;
        if ((lane & 15) == 0 && orow < rows_wg) {
          if (KS == 1) store_out(w.y, base + orow, v * st, a.ydt);
          else part[ks * kGemvMaxRpw + orow] = v;
        }
      }
    }
  }
  if (KS > 1) {
    __syncthreads();
    for (int r = threadIdx.x; r < rows_wg; r += 256) {
      float v = 0.0f;
#pragma unroll
      for (int q = 0; q < KS; q++) v += part[q * kGemvMaxRpw + r];
      store_out(w.y, base + r, v * st, a.ydt);
    }
  }
}

size_t gemv_ws_bytes(int64_t, int64_t) { return 0; }

struct GemvPlan {
  int ks, cpl, nq, rpwv, rpw;
  int64_t grid;
};

template <typename XT, int UNIT, int CPL, int KS, int NQ>
static hipError_t launch_cfg(GemvArgs a, const GemvPlan& p, bool f16s, hipStream_t stream) {
  a.rpw = p.rpw;
  a.rpwv = p.rpwv;
  if constexpr (UNIT == 2) {
    if (f16s) {
      hipLaunchKernelGGL((gemv_kernel<XT, UNIT, CPL, KS, NQ, true, true>), dim3((unsigned)p.grid), dim3(256),
                         0, stream, a);
      return hipGetLastError();
    }
  }
  // wide scale loads need the scale row stride (K / 16 bytes) to keep 4 * UNIT alignment
  if ((a.k / 16) % (4 * UNIT) == 0)
    hipLaunchKernelGGL((gemv_kernel<XT, UNIT, CPL, KS, NQ, true, false>), dim3((unsigned)p.grid), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((gemv_kernel<XT, UNIT, CPL, KS, NQ, false, false>), dim3((unsigned)p.grid), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

// Launch sizing (the CDNA counterpart of the pages' SM-launch trimming).  K is
// split over KS waves when a lane would otherwise hold more than two chunks of
// x; each row group then gets a run of whole row quads, sized so that about
// wg_per_cu workgroups land on each CU, and never more workgroups than the
// rows need.
//
// The untrimmed plan (RAZER_FLAG_UNTRIMMED_PLAN) instead splits K over as many
// waves as keep every lane busy (up to 4) and gives each row group one quad,
// so the launch has as many workgroups as the rows allow.
static GemvPlan plan_gemv(int64_t n, int64_t nchunk, int cus, int wg_per_cu, bool untrimmed = false) {
  GemvPlan p;
  p.ks = nchunk <= 64 ? 1 : nchunk <= 128 ? 2 : 4;
  if (untrimmed) p.ks = nchunk >= 256 ? 4 : nchunk >= 128 ? 2 : 1;
  const int64_t per_lane = (nchunk + 64LL * p.ks - 1) / (64LL * p.ks);
  p.cpl = per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : per_lane <= 4 ? 4 : per_lane <= 8 ? 8 : 16;
  p.nq = 1;
  const int rw = 4 / p.ks;
  const int64_t groups = (int64_t)cus * wg_per_cu * rw;
  int64_t rpwv = (n + groups - 1) / groups;
  rpwv = (rpwv + 3) / 4 * 4;
  if (rpwv * rw > kGemvMaxRpw) rpwv = kGemvMaxRpw / rw;
  if (untrimmed) rpwv = 4;
  p.rpwv = (int)rpwv;
  p.rpw = (int)(rpwv * rw);
  p.grid = (n + p.rpw - 1) / p.rpw;
  return p;
}

template <typename XT, int UNIT>
static hipError_t dispatch(const GemvArgs& a, const GemvPlan& p, bool f16s, hipStream_t stream) {
#define RZ_CASE(C_, K_, Q_) \
  if (p.cpl == C_ && p.ks == K_ && p.nq == Q_) return launch_cfg<XT, UNIT, C_, K_, Q_>(a, p, f16s, stream);
  RZ_CASE(1, 1, 1) RZ_CASE(1, 2, 1) RZ_CASE(1, 4, 1) RZ_CASE(2, 4, 1) RZ_CASE(4, 4, 1)
  RZ_CASE(8, 4, 1)
  if constexpr (UNIT == 1) {
    RZ_CASE(16, 4, 1)  // 16-element chunks with K up to 65536
  }
#undef RZ_CASE
  return hipErrorInvalidValue;
}

// Weights that go to the MFMA small-batch kernel instead: long rows (K above
// 8192) on up to 4096 rows, where its K split keeps enough waves busy
// (measured faster there only); both the default layout and 128-element
// blocks with FP16 scales.
static bool gemv_to_smallm(const PackedView& w) {
  const bool layout_ok = default_layout(w) || (w.blog2 == 7 && w.sfmt == 1);
  return layout_ok && w.rows <= 4096 && w.cols > 8192 && smallm_supported(1, w.rows, w.cols);
}

hipError_t launch_gemv_group(const void* x, int x_dtype, const PackedView* w, void* const* y,
                             int count, int y_dtype, hipStream_t stream) {
  if (count < 1 || count > kGemvGroupMax) return hipErrorInvalidValue;
  // one layout per launch: 16-element blocks with byte scales, or 128-element
  // blocks with FP16 scales (K a multiple of 128)
  const bool f16s = !default_layout(w[0]);
  for (int g = 0; g < count; g++)
    if (default_layout(w[g]) == f16s || (f16s && (w[g].blog2 != 7 || w[g].sfmt != 1)))
      return hipErrorInvalidValue;
  // members for the small-batch kernel, and empty ones, are launched on their own
  GemvArgs a;
  a.x = x;
  a.count = 0;
  a.k = w[0].cols;
  a.ydt = y_dtype;
  int64_t n_total = 0;
  for (int g = 0; g < count; g++) {
    if (w[g].rows <= 0) continue;
    if (gemv_to_smallm(w[g])) {
      const hipError_t e = launch_smallm(x, x_dtype, 1, w[g], y[g], y_dtype, stream);
      if (e != hipSuccess) return e;
      continue;
    }
    GemvWeight& m = a.w[a.count++];
    m.codes = w[g].codes;
    m.scales = w[g].scales;
    m.ts = w[g].tensor_scale;
    m.y = y[g];
    m.n = w[g].rows;
    m.kind = w[g].kind;
    m.m0 = 6.0f + 0.5f * (float)w[g].off_half[0];
    m.m1 = 6.0f + 0.5f * (float)w[g].off_half[w[g].kind == kWeight ? 1 : 0];
    n_total += m.n;
  }
  if (a.count == 0) return hipSuccess;
  bool untrimmed = false;
  for (int g = 0; g < count; g++) untrimmed = untrimmed || (w[g].flags & kFlagUntrimmed);
  // the untrimmed plan takes 16-element chunks (twice the K split) where the layout allows
  const bool unit2 = a.k % 32 == 0 && (f16s || !untrimmed);
  if (f16s && !unit2) return hipErrorInvalidValue;
  a.nchunk = a.k / (unit2 ? 32 : 16);
  // one plan for the summed rows; each weight gets whole workgroups of it
  GemvPlan p = plan_gemv(n_total, a.nchunk, device_cu_count(), 8, untrimmed);
  int64_t wg = 0;
  for (int g = 0; g < a.count; g++) {
    a.w[g].wg0 = (int)wg;
    wg += (a.w[g].n + p.rpw - 1) / p.rpw;
  }
  for (int g = a.count; g < kGemvGroupMax; g++) a.w[g] = a.w[0];
  p.grid = wg;
  if (x_dtype == kF16)
    return unit2 ? dispatch<_Float16, 2>(a, p, f16s, stream) : dispatch<_Float16, 1>(a, p, f16s, stream);
  return unit2 ? dispatch<__bf16, 2>(a, p, f16s, stream) : dispatch<__bf16, 1>(a, p, f16s, stream);
}

hipError_t launch_gemv(const void* x, int x_dtype, const PackedView& w, void* y, int y_dtype,
                       void*, size_t, hipStream_t stream) {
  return launch_gemv_group(x, x_dtype, &w, &y, 1, y_dtype, stream);
}

}  // namespace rz
