// rz_api.cpp -- the extern "C" entry points of librazer (see include/librazer.h).
//
// Host-side argument checks happen here, synchronously, before anything is
// enqueued; then the launchers in the kernel translation units are called on
// the caller's stream.  No allocation, no synchronisation, no exceptions cross
// the ABI.
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include "../../include/librazer.h"
#include "rz_launch.h"

namespace rz {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const int slot = dev & 63;
  int v = cache[slot].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
    cu = 256;
  cache[slot].store(cu, std::memory_order_relaxed);
  return cu;
}

}  // namespace rz

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool dtype_ok(int dt) { return dt == RAZER_F32 || dt == RAZER_F16 || dt == RAZER_BF16; }

// Shape and offset checks shared by every call that reads or writes a packed tensor.
razer_status check_packed(const razer_packed* p, bool need_data) {
  if (!p) return RAZER_E_INVALID;
  if (p->kind != RAZER_WEIGHT && p->kind != RAZER_ACT) return RAZER_E_INVALID;
  const int blog2 = p->block_log2 ? p->block_log2 : 4;
  if (blog2 < 4 || blog2 > 7) return RAZER_E_INVALID;
  if (p->scale_fmt != RAZER_SCALE_BYTE && p->scale_fmt != RAZER_SCALE_F16) return RAZER_E_INVALID;
  if (p->scale_fmt == RAZER_SCALE_F16 && p->kind != RAZER_WEIGHT) return RAZER_E_INVALID;
  if (p->rows < 0 || p->cols < 0 || p->cols % (1 << blog2) != 0) return RAZER_E_INVALID;
  if (p->cols > 0 && p->rows > INT64_MAX / 2 / p->cols) return RAZER_E_INVALID;
  const int npairs = p->kind == RAZER_WEIGHT ? 2 : 1;
  for (int i = 0; i < npairs; i++)
    if (p->sv_off_half[i] < -7 || p->sv_off_half[i] > 7) return RAZER_E_INVALID;
  if (!p->tensor_scale || !aligned(p->tensor_scale, 4)) return RAZER_E_INVALID;
  if (need_data && p->rows * p->cols > 0) {
    if (!p->codes || !p->scales) return RAZER_E_INVALID;
    if (!aligned(p->codes, 16) || !aligned(p->scales, 4)) return RAZER_E_INVALID;
  }
  return RAZER_OK;
}

rz::PackedView view_of(const razer_packed* p) {
  rz::PackedView v;
  v.kind = p->kind;
  v.flags = p->flags;
  v.rows = p->rows;
  v.cols = p->cols;
  v.off_half[0] = p->sv_off_half[0];
  v.off_half[1] = p->kind == RAZER_WEIGHT ? p->sv_off_half[1] : p->sv_off_half[0];
  v.blog2 = p->block_log2 ? p->block_log2 : 4;
  v.sfmt = p->scale_fmt;
  v.codes = p->codes;
  v.scales = p->scales;
  v.tensor_scale = p->tensor_scale;
  return v;
}

static_assert(RAZER_FLAG_NO_REMAP == rz::kFlagNoRemap && RAZER_FLAG_FOUR_OVER_SIX == rz::kFlagFourOverSix &&
                  RAZER_FLAG_UNTRIMMED_PLAN == rz::kFlagUntrimmed && RAZER_FLAG_RESCALE_LARGE_SV == rz::kFlagRescale,
              "flag values");

constexpr uint32_t kEncoderFlags = RAZER_FLAG_NO_REMAP | RAZER_FLAG_FOUR_OVER_SIX | RAZER_FLAG_RESCALE_LARGE_SV;

// The encoder flags a packed output may carry: the rescale mode exists for
// 16-element blocks with byte scales only.
razer_status check_encoder_flags(const razer_packed* out) {
  if (out->flags & ~kEncoderFlags) return RAZER_E_INVALID;
  if ((out->flags & RAZER_FLAG_RESCALE_LARGE_SV) && !((out->block_log2 == 0 || out->block_log2 == 4) &&
                                                      out->scale_fmt == RAZER_SCALE_BYTE))
    return RAZER_E_UNSUPPORTED;
  return RAZER_OK;
}

// The product kernels read 16-element blocks with byte scales; the GEMV and
// razer_gemm also read 128-element blocks with FP16 scales.
bool product_layout(const razer_packed* p) {
  return (p->block_log2 == 0 || p->block_log2 == 4) && p->scale_fmt == RAZER_SCALE_BYTE;
}
bool gemv_layout(const razer_packed* p) {
  return product_layout(p) || (p->block_log2 == 7 && p->scale_fmt == RAZER_SCALE_F16);
}

razer_status status_of(hipError_t e) { return e == hipSuccess ? RAZER_OK : RAZER_E_HIP; }

razer_status quantize_common(const void* x, razer_dtype dt, const razer_packed* out, void* ws,
                             size_t ws_bytes, void* stream, int kind) {
  razer_status s = check_packed(out, true);
  if (s != RAZER_OK) return s;
  s = check_encoder_flags(out);
  if (s != RAZER_OK) return s;
  if (out->kind != kind || !dtype_ok(dt)) return RAZER_E_INVALID;
  const int64_t n = out->rows * out->cols;
  if (n > 0 && (!x || !aligned(x, 16))) return RAZER_E_INVALID;
  const size_t need = rz::quantize_ws_bytes();
  if (!ws || ws_bytes < need || !aligned(ws, 4)) return RAZER_E_INVALID;
  return status_of(rz::launch_quantize(x, dt, view_of(out), ws, (hipStream_t)stream));
}

constexpr int64_t kGemvMaxK = 65536;  // each lane holds at most 8 x 32 or 16 x 16 elements of x

}  // namespace

extern "C" {

razer_status razer_quantize_weight(const void* w, razer_dtype w_dt, const razer_packed* out,
                                   void* ws, size_t ws_bytes, void* stream) {
  return quantize_common(w, w_dt, out, ws, ws_bytes, stream, RAZER_WEIGHT);
}

razer_status razer_quantize_act(const void* x, razer_dtype x_dt, const razer_packed* out,
                                void* ws, size_t ws_bytes, void* stream) {
  return quantize_common(x, x_dt, out, ws, ws_bytes, stream, RAZER_ACT);
}

razer_status razer_quantize_act_noalloc(const void* x, razer_dtype x_dt, const razer_packed* out,
                                        void* stream) {
  razer_status s = check_packed(out, true);
  if (s != RAZER_OK) return s;
  s = check_encoder_flags(out);
  if (s != RAZER_OK) return s;
  if (out->kind != RAZER_ACT || !dtype_ok(x_dt)) return RAZER_E_INVALID;
  const int64_t n = out->rows * out->cols;
  if (n > 0 && (!x || !aligned(x, 16))) return RAZER_E_INVALID;
  if (rz::quantize_ws_bytes() > rz::noalloc_scratch_bytes()) return RAZER_E_UNSUPPORTED;
  return status_of(rz::launch_quantize_noalloc(x, x_dt, view_of(out), (hipStream_t)stream));
}

razer_status razer_dequant(const razer_packed* t, void* out, razer_dtype out_dt, void* stream) {
  razer_status s = check_packed(t, true);
  if (s != RAZER_OK) return s;
  if (!dtype_ok(out_dt)) return RAZER_E_INVALID;
  if (t->rows * t->cols == 0) return RAZER_OK;
  if (!out || !aligned(out, 16)) return RAZER_E_INVALID;
  return status_of(rz::launch_dequant(view_of(t), out, out_dt, (hipStream_t)stream));
}

razer_status razer_gemv(const void* x, razer_dtype x_dt, const razer_packed* w, void* y,
                        razer_dtype y_dt, void* ws, size_t ws_bytes, void* stream) {
  razer_status s = check_packed(w, true);
  if (s != RAZER_OK) return s;
  if (!dtype_ok(x_dt) || !dtype_ok(y_dt)) return RAZER_E_INVALID;
  if (x_dt == RAZER_F32 || !gemv_layout(w)) return RAZER_E_UNSUPPORTED;
  if (w->cols > kGemvMaxK) return RAZER_E_UNSUPPORTED;
  if (w->rows == 0) return RAZER_OK;
  if (!y || !aligned(y, 16)) return RAZER_E_INVALID;
  if (w->cols > 0 && (!x || !aligned(x, 16))) return RAZER_E_INVALID;
  const size_t need = rz::gemv_ws_bytes(w->rows, w->cols);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 4))) return RAZER_E_INVALID;
  return status_of(rz::launch_gemv(x, x_dt, view_of(w), y, y_dt, ws, ws_bytes, (hipStream_t)stream));
}

razer_status razer_gemv_group(const void* x, razer_dtype x_dt, const razer_packed* const* w,
                              void* const* y, int count, razer_dtype y_dt, void* stream) {
  if (count < 1 || count > RAZER_GEMV_GROUP_MAX || !w || !y) return RAZER_E_INVALID;
  if (!dtype_ok(x_dt) || !dtype_ok(y_dt)) return RAZER_E_INVALID;
  rz::PackedView v[RAZER_GEMV_GROUP_MAX];
  void* yy[RAZER_GEMV_GROUP_MAX];
  for (int g = 0; g < count; g++) {
    razer_status s = check_packed(w[g], true);
    if (s != RAZER_OK) return s;
    if (w[g]->cols != w[0]->cols) return RAZER_E_INVALID;
    if (w[g]->rows > 0 && (!y[g] || !aligned(y[g], 16))) return RAZER_E_INVALID;
    v[g] = view_of(w[g]);
    yy[g] = y[g];
  }
  for (int g = 0; g < count; g++)
    if (!gemv_layout(w[g]) || product_layout(w[g]) != product_layout(w[0])) return RAZER_E_UNSUPPORTED;
  if (x_dt == RAZER_F32) return RAZER_E_UNSUPPORTED;
  if (w[0]->cols > kGemvMaxK) return RAZER_E_UNSUPPORTED;
  if (w[0]->cols > 0 && (!x || !aligned(x, 16))) return RAZER_E_INVALID;
  return status_of(rz::launch_gemv_group(x, x_dt, v, yy, count, y_dt, (hipStream_t)stream));
}

razer_status razer_gemm(const void* x, razer_dtype x_dt, int64_t m, const razer_packed* w, void* y,
                        razer_dtype y_dt, void* ws, size_t ws_bytes, void* stream) {
  razer_status s = check_packed(w, true);
  if (s != RAZER_OK) return s;
  if (!dtype_ok(x_dt) || !dtype_ok(y_dt) || m < 0) return RAZER_E_INVALID;
  if (x_dt == RAZER_F32 || !gemv_layout(w)) return RAZER_E_UNSUPPORTED;
  if (m == 0 || w->rows == 0) return RAZER_OK;
  if (m == 1) return razer_gemv(x, x_dt, w, y, y_dt, ws, ws_bytes, stream);
  if (!y || !aligned(y, 16)) return RAZER_E_INVALID;
  if (w->cols > 0 && (!x || !aligned(x, 16))) return RAZER_E_INVALID;
  if (m > INT64_MAX / 2 / (w->rows > w->cols ? w->rows : (w->cols ? w->cols : 1)))
    return RAZER_E_INVALID;
  const size_t need = rz::gemm_ws_need(m, w->rows, w->cols, !product_layout(w),
                                       (w->flags & RAZER_FLAG_UNTRIMMED_PLAN) != 0);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 4))) return RAZER_E_INVALID;
  return status_of(
      rz::launch_gemm(x, x_dt, m, view_of(w), y, y_dt, ws, ws_bytes, (hipStream_t)stream));
}

razer_status razer_gemm_w4a4(const razer_packed* x, const razer_packed* w, void* y, razer_dtype y_dt,
                             void* ws, size_t ws_bytes, void* stream) {
  razer_status s = check_packed(x, true);
  if (s != RAZER_OK) return s;
  s = check_packed(w, true);
  if (s != RAZER_OK) return s;
  if (!dtype_ok(y_dt) || x->cols != w->cols) return RAZER_E_INVALID;
  if (!product_layout(x) || !product_layout(w)) return RAZER_E_UNSUPPORTED;
  if (x->rows == 0 || w->rows == 0) return RAZER_OK;
  if (x->cols == 0) return RAZER_E_UNSUPPORTED;
  if (w->cols > kGemvMaxK && x->rows == 1) return RAZER_E_UNSUPPORTED;
  if (!y || !aligned(y, 16)) return RAZER_E_INVALID;
  if (x->rows > INT64_MAX / 4 / (w->rows > w->cols ? w->rows : w->cols)) return RAZER_E_INVALID;
  const size_t need = rz::gemm_w4a4_ws_bytes(x->rows, w->rows, w->cols);
  if (!ws || ws_bytes < need || !aligned(ws, 256)) return RAZER_E_INVALID;
  return status_of(rz::launch_gemm_w4a4(view_of(x), view_of(w), y, y_dt, ws, ws_bytes, (hipStream_t)stream));
}

razer_status razer_weight_offset_sse(const void* w, razer_dtype w_dt, int64_t rows, int64_t cols,
                                     int off0_half, double* sse, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (!dtype_ok(w_dt) || rows < 0 || cols < 0 || cols % 16 != 0) return RAZER_E_INVALID;
  if (cols > 0 && rows > INT64_MAX / 2 / cols) return RAZER_E_INVALID;
  if (off0_half < -7 || off0_half > 7) return RAZER_E_INVALID;
  if (!sse || !aligned(sse, 8)) return RAZER_E_INVALID;
  const int64_t n = rows * cols;
  if (n > 0 && (!w || !aligned(w, 16))) return RAZER_E_INVALID;
  const size_t need = rz::offset_search_ws_bytes(n);
  if (!ws || ws_bytes < need || !aligned(ws, 8)) return RAZER_E_INVALID;
  return status_of(rz::launch_offset_search(w, w_dt, rows, cols, off0_half, sse, ws, (hipStream_t)stream));
}

size_t razer_workspace_bytes(int op, int64_t m, int64_t n, int64_t k) {
  switch (op) {
    case RAZER_OP_QUANTIZE_WEIGHT:
    case RAZER_OP_QUANTIZE_ACT:
      return rz::quantize_ws_bytes();
    case RAZER_OP_GEMV:
      return rz::gemv_ws_bytes(n, k);
    case RAZER_OP_GEMM:
      return m <= 1 ? rz::gemv_ws_bytes(n, k) : rz::gemm_ws_bytes(m, n, k);
    case RAZER_OP_GEMM_UNTRIMMED: {
      if (m <= 1) return rz::gemv_ws_bytes(n, k);
      const size_t a = rz::gemm_ws_need(m, n, k, false, true), b = rz::gemm_ws_need(m, n, k, true, true);
      return a > b ? a : b;
    }
    case RAZER_OP_GEMM_W4A4:
      return rz::gemm_w4a4_ws_bytes(m, n, k);
    case RAZER_OP_OFFSET_SEARCH:
      return (n < 0 || k < 0) ? 0 : rz::offset_search_ws_bytes(n * k);
    default:
      return 0;
  }
}

const char* razer_status_string(razer_status s) {
  switch (s) {
    case RAZER_OK: return "RAZER_OK";
    case RAZER_E_INVALID: return "RAZER_E_INVALID: invalid argument";
    case RAZER_E_UNSUPPORTED: return "RAZER_E_UNSUPPORTED: unsupported combination";
    case RAZER_E_HIP: return "RAZER_E_HIP: kernel launch failed";
    default: return "unknown razer_status";
  }
}

}  // extern "C"
