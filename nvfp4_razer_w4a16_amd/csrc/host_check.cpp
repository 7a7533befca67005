// host_check.cpp -- test infrastructure only (tests/test_sanitizers.py): a
// host build of rz_api.cpp, the C ABI's argument checks, linked against stub
// launchers instead of the kernels, run under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every entry point is called with rejected and
// with accepted arguments (fake, never dereferenced device addresses); the
// stubs count the launches an accepted call reaches.  Exit status 0 and no
// sanitizer report means clean.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>

#include "../../include/librazer.h"
#include "rz_launch.h"

namespace {
int g_launches = 0;
hipError_t counted() {
  g_launches++;
  return hipSuccess;
}
}  // namespace

namespace rz {
size_t quantize_ws_bytes() { return kAmaxMaxPartials * sizeof(uint32_t); }
hipError_t launch_quantize(const void*, int, const PackedView&, void*, hipStream_t) { return counted(); }
size_t noalloc_scratch_bytes() { return 4096; }
hipError_t launch_quantize_noalloc(const void*, int, const PackedView&, hipStream_t) { return counted(); }
size_t offset_search_ws_bytes(int64_t n) { return 4096 + (size_t)(n > 0 ? 1024 : 0) * 15 * 8; }
hipError_t launch_offset_search(const void*, int, int64_t, int64_t, int, double*, void*, hipStream_t) {
  return counted();
}
hipError_t launch_dequant(const PackedView&, void*, int, hipStream_t) { return counted(); }
hipError_t launch_dequant_unscaled(const PackedView&, void*, int, hipStream_t) { return counted(); }
size_t gemm_w4a4_ws_bytes(int64_t m, int64_t n, int64_t k) {
  return (size_t)(m * k * 2 + m * n * 4 + 256);
}
hipError_t launch_gemm_w4a4(const PackedView&, const PackedView&, void*, int, void*, size_t, hipStream_t) {
  return counted();
}
size_t gemv_ws_bytes(int64_t, int64_t) { return 0; }
hipError_t launch_gemv_group(const void*, int, const PackedView*, void* const*, int, int, hipStream_t) {
  return counted();
}
bool gemm_prefill_fits(int64_t m, int64_t k, int) { return m >= 256 && k % 64 == 0; }
hipError_t launch_gemm_prefill_scaled(const void*, int, int64_t, const PackedView&, void*, int, const float*,
                                      hipStream_t) {
  return counted();
}
hipError_t launch_gemv(const void*, int, const PackedView&, void*, int, void*, size_t, hipStream_t) {
  return counted();
}
bool smallm_supported(int64_t m, int64_t, int64_t k) { return m >= 1 && m <= 4 && k % 256 == 0; }
hipError_t launch_smallm(const void*, int, int64_t, const PackedView&, void*, int, hipStream_t) {
  return counted();
}
size_t gemm_ws_bytes(int64_t m, int64_t n, int64_t) { return (size_t)(4 * m * n * 4); }
size_t gemm_ws_need(int64_t m, int64_t n, int64_t k, bool, bool) { return gemm_ws_bytes(m, n, k); }
hipError_t launch_gemm(const void*, int, int64_t, const PackedView&, void*, int, void*, size_t, hipStream_t) {
  return counted();
}
}  // namespace rz

namespace {

int g_fail = 0;
void expect(razer_status got, razer_status want, const char* what) {
  if (got != want) {
    fprintf(stderr, "host_check: %s: got %d, want %d\n", what, (int)got, (int)want);
    g_fail = 1;
  }
}

void* fake(uintptr_t a) { return (void*)a; }

razer_packed packed(int kind, int64_t rows, int64_t cols) {
  razer_packed p = {};
  p.kind = kind;
  p.rows = rows;
  p.cols = cols;
  p.sv_off_half[0] = -2;
  p.sv_off_half[1] = 4;
  p.codes = (uint8_t*)fake(0x100000);
  p.scales = (uint8_t*)fake(0x200000);
  p.tensor_scale = (float*)fake(0x300000);
  return p;
}

}  // namespace

int main() {
  void* x = fake(0x400000);
  void* y = fake(0x500000);
  void* ws = fake(0x600000);
  const size_t big = (size_t)1 << 40;
  razer_packed w = packed(RAZER_WEIGHT, 64, 256), a = packed(RAZER_ACT, 8, 256);

  // encoders
  expect(razer_quantize_weight(x, RAZER_F32, &w, ws, big, nullptr), RAZER_OK, "quantize_weight ok");
  expect(razer_quantize_weight(nullptr, RAZER_F32, &w, ws, big, nullptr), RAZER_E_INVALID, "null x");
  expect(razer_quantize_weight(fake(0x400004), RAZER_F32, &w, ws, big, nullptr), RAZER_E_INVALID, "misaligned x");
  expect(razer_quantize_weight(x, RAZER_F32, &w, ws, 16, nullptr), RAZER_E_INVALID, "small workspace");
  expect(razer_quantize_weight(x, (razer_dtype)9, &w, ws, big, nullptr), RAZER_E_INVALID, "bad dtype");
  expect(razer_quantize_weight(x, RAZER_F32, nullptr, ws, big, nullptr), RAZER_E_INVALID, "null out");
  expect(razer_quantize_weight(x, RAZER_F32, &a, ws, big, nullptr), RAZER_E_INVALID, "wrong kind");
  expect(razer_quantize_act(x, RAZER_BF16, &a, ws, big, nullptr), RAZER_OK, "quantize_act ok");
  expect(razer_quantize_act_noalloc(x, RAZER_BF16, &a, nullptr), RAZER_OK, "noalloc ok");
  expect(razer_quantize_act_noalloc(x, RAZER_BF16, &w, nullptr), RAZER_E_INVALID, "noalloc wrong kind");
  {
    razer_packed bad = w;
    bad.sv_off_half[1] = 8;
    expect(razer_quantize_weight(x, RAZER_F32, &bad, ws, big, nullptr), RAZER_E_INVALID, "offset 8");
    bad = w;
    bad.cols = 250;
    expect(razer_quantize_weight(x, RAZER_F32, &bad, ws, big, nullptr), RAZER_E_INVALID, "cols % 16");
    bad = w;
    bad.rows = INT64_MAX / 4;
    bad.cols = 1024;
    expect(razer_quantize_weight(x, RAZER_F32, &bad, ws, big, nullptr), RAZER_E_INVALID, "size overflow");
    bad = w;
    bad.flags = 64;
    expect(razer_quantize_weight(x, RAZER_F32, &bad, ws, big, nullptr), RAZER_E_INVALID, "unknown flag");
    bad = w;
    bad.block_log2 = 9;
    expect(razer_quantize_weight(x, RAZER_F32, &bad, ws, big, nullptr), RAZER_E_INVALID, "block_log2 9");
    bad = a;
    bad.scale_fmt = RAZER_SCALE_F16;
    expect(razer_quantize_act(x, RAZER_BF16, &bad, ws, big, nullptr), RAZER_E_INVALID, "act FP16 scales");
    bad = w;
    bad.codes = (uint8_t*)fake(0x100008);
    expect(razer_quantize_weight(x, RAZER_F32, &bad, ws, big, nullptr), RAZER_E_INVALID, "misaligned codes");
  }

  // decoder and products
  expect(razer_dequant(&w, y, RAZER_BF16, nullptr), RAZER_OK, "dequant ok");
  expect(razer_dequant(&w, nullptr, RAZER_BF16, nullptr), RAZER_E_INVALID, "dequant null out");
  expect(razer_gemv(x, RAZER_F16, &w, y, RAZER_F32, nullptr, 0, nullptr), RAZER_OK, "gemv ok");
  expect(razer_gemv(x, RAZER_F32, &w, y, RAZER_F32, nullptr, 0, nullptr), RAZER_E_UNSUPPORTED, "gemv f32 x");
  expect(razer_gemv(x, RAZER_F16, &w, fake(0x500004), RAZER_F32, nullptr, 0, nullptr), RAZER_E_INVALID,
         "gemv misaligned y");
  {
    razer_packed longk = packed(RAZER_WEIGHT, 4, 65536 + 16);
    expect(razer_gemv(x, RAZER_F16, &longk, y, RAZER_F32, nullptr, 0, nullptr), RAZER_E_UNSUPPORTED,
           "gemv K above 65536");
  }
  {
    const razer_packed* ws2[2] = {&w, &w};
    void* ys[2] = {y, y};
    expect(razer_gemv_group(x, RAZER_F16, ws2, ys, 2, RAZER_F16, nullptr), RAZER_OK, "group ok");
    expect(razer_gemv_group(x, RAZER_F16, ws2, ys, 0, RAZER_F16, nullptr), RAZER_E_INVALID, "group count 0");
    expect(razer_gemv_group(x, RAZER_F16, ws2, ys, 5, RAZER_F16, nullptr), RAZER_E_INVALID, "group count 5");
    razer_packed other = packed(RAZER_WEIGHT, 64, 512);
    const razer_packed* mixed[2] = {&w, &other};
    expect(razer_gemv_group(x, RAZER_F16, mixed, ys, 2, RAZER_F16, nullptr), RAZER_E_INVALID, "group unequal K");
  }
  expect(razer_gemm(x, RAZER_BF16, 8, &w, y, RAZER_BF16, ws, big, nullptr), RAZER_OK, "gemm ok");
  expect(razer_gemm(x, RAZER_BF16, 8, &w, y, RAZER_BF16, ws, 4, nullptr), RAZER_E_INVALID, "gemm small ws");
  expect(razer_gemm(x, RAZER_BF16, -1, &w, y, RAZER_BF16, ws, big, nullptr), RAZER_E_INVALID, "gemm m < 0");
  expect(razer_gemm(x, RAZER_BF16, INT64_MAX / 2, &w, y, RAZER_BF16, ws, big, nullptr), RAZER_E_INVALID,
         "gemm m overflow");
  expect(razer_gemm(x, RAZER_BF16, 0, &w, y, RAZER_BF16, ws, big, nullptr), RAZER_OK, "gemm m 0");
  expect(razer_gemm_w4a4(&a, &w, y, RAZER_BF16, ws, big, nullptr), RAZER_OK, "w4a4 ok");
  expect(razer_gemm_w4a4(&a, &w, y, RAZER_BF16, fake(0x600010), big, nullptr), RAZER_E_INVALID,
         "w4a4 misaligned ws");
  {
    double* sse = (double*)fake(0x700000);
    expect(razer_weight_offset_sse(x, RAZER_F32, 64, 256, -2, sse, ws, big, nullptr), RAZER_OK, "offset ok");
    expect(razer_weight_offset_sse(x, RAZER_F32, 64, 256, 8, sse, ws, big, nullptr), RAZER_E_INVALID,
           "offset off0 8");
    expect(razer_weight_offset_sse(x, RAZER_F32, 64, 250, -2, sse, ws, big, nullptr), RAZER_E_INVALID,
           "offset cols % 16");
  }
  for (int s = 0; s < 5; s++)
    if (!razer_status_string((razer_status)s)) g_fail = 1;
  for (int op = -1; op < 8; op++) (void)razer_workspace_bytes(op, 4, 64, 256);
  (void)razer_workspace_bytes(RAZER_OP_OFFSET_SEARCH, 0, -1, 16);
  if (g_launches != 9) {
    fprintf(stderr, "host_check: %d launches reached, want 9\n", g_launches);
    g_fail = 1;
  }
  printf("host_check: %s (%d launches)\n", g_fail ? "FAILED" : "ok", g_launches);
  return g_fail;
}
