"""C-ABI checks that need no GPU: the library loads, exports every function
include/librazer.h declares, and rejects bad arguments on the host before any
HIP call."""
import ctypes
import os
import re

import pytest

import nvfp4_razer_w4a16_amd as rz

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "librazer.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(razer_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = _declared_functions()
    for n in ("razer_quantize_weight", "razer_quantize_act", "razer_dequant", "razer_gemv",
              "razer_gemm"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = rz.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    assert set(rz.EXPORTED) <= set(_declared_functions())


def test_struct_layout_matches_header():
    # int32 kind, uint32 flags, int64 rows, int64 cols, int8[2] offsets, uint8 block_log2,
    # uint8 scale_fmt, 4 reserved, 3 pointers
    assert ctypes.sizeof(rz.razer_packed) == 4 + 4 + 8 + 8 + 8 + 3 * 8
    assert rz.razer_packed.block_log2.offset == 26 and rz.razer_packed.scale_fmt.offset == 27
    assert rz.razer_packed.codes.offset == 32


def test_status_strings():
    assert rz.razer_status_string(rz.RAZER_OK) == "RAZER_OK"
    assert "invalid" in rz.razer_status_string(rz.RAZER_E_INVALID)
    assert "unknown" in rz.razer_status_string(99)


def test_workspace_sizes():
    assert rz.razer_workspace_bytes(rz.RAZER_OP_QUANTIZE_WEIGHT, 0, 256, 1024) >= 4096
    assert rz.razer_workspace_bytes(rz.RAZER_OP_QUANTIZE_ACT, 4096, 0, 8192) >= 4096
    assert rz.razer_workspace_bytes(99, 1, 1, 1) == 0


def _packed(kind=rz.RAZER_WEIGHT, rows=4, cols=32, off=(-2, 4), codes=0x1000, scales=0x2000,
            ts=0x3000):
    s = rz.razer_packed()
    s.kind, s.flags, s.rows, s.cols = kind, 0, rows, cols
    s.sv_off_half[0], s.sv_off_half[1] = off
    s.codes, s.scales, s.tensor_scale = codes, scales, ts
    return s


FAKE_X = ctypes.c_void_p(0x4000)   # never dereferenced: every case fails host checks
FAKE_WS = ctypes.c_void_p(0x5000)


@pytest.mark.parametrize("mutate", [
    lambda s: setattr(s, "cols", 24),                  # cols % 16 != 0
    lambda s: setattr(s, "rows", -1),
    lambda s: s.sv_off_half.__setitem__(0, 8),         # offset outside [-7, 7]
    lambda s: s.sv_off_half.__setitem__(1, -8),
    lambda s: setattr(s, "codes", None),
    lambda s: setattr(s, "scales", None),
    lambda s: setattr(s, "tensor_scale", None),
    lambda s: setattr(s, "codes", 0x1008),             # misaligned codes
    lambda s: setattr(s, "kind", rz.RAZER_ACT),        # wrong kind for the weight encoder
    lambda s: setattr(s, "kind", 7),
    lambda s: setattr(s, "block_log2", 3),             # block sizes are 16..128
    lambda s: setattr(s, "block_log2", 8),
    lambda s: setattr(s, "block_log2", 6),             # cols (32) not a multiple of 64
    lambda s: setattr(s, "scale_fmt", 2),
    lambda s: setattr(s, "flags", 4),                  # unknown encoder flag bit
    lambda s: setattr(s, "flags", 16),
    lambda s: setattr(s, "flags", 0x80000002),
])
def test_quantize_weight_rejects_bad_packed(mutate):
    s = _packed()
    mutate(s)
    st = rz.lib().razer_quantize_weight(FAKE_X, rz.RAZER_F32, ctypes.byref(s), FAKE_WS, 4096, None)
    assert st == rz.RAZER_E_INVALID


def test_rescale_flag_only_on_the_default_layout():
    # RAZER_FLAG_RESCALE_LARGE_SV encodes 16-element blocks with byte scales;
    # other layouts are refused before any launch
    L = rz.lib()
    for blog2, sfmt in ((5, rz.RAZER_SCALE_BYTE), (7, rz.RAZER_SCALE_F16)):
        s = _packed(cols=128)
        s.flags, s.block_log2, s.scale_fmt = rz.RAZER_FLAG_RESCALE_LARGE_SV, blog2, sfmt
        st = L.razer_quantize_weight(FAKE_X, rz.RAZER_F32, ctypes.byref(s), FAKE_WS, 4096, None)
        assert st == rz.RAZER_E_UNSUPPORTED
    a = _packed(kind=rz.RAZER_ACT, cols=64)
    a.flags, a.block_log2 = rz.RAZER_FLAG_RESCALE_LARGE_SV, 6
    assert L.razer_quantize_act(FAKE_X, rz.RAZER_BF16, ctypes.byref(a), FAKE_WS, 4096, None) == rz.RAZER_E_UNSUPPORTED
    assert L.razer_quantize_act_noalloc(FAKE_X, rz.RAZER_BF16, ctypes.byref(a), None) == rz.RAZER_E_UNSUPPORTED


def test_quantize_rejects_bad_buffers():
    L = rz.lib()
    s = _packed()
    assert L.razer_quantize_weight(None, rz.RAZER_F32, ctypes.byref(s), FAKE_WS, 4096, None) == rz.RAZER_E_INVALID
    assert L.razer_quantize_weight(ctypes.c_void_p(0x4004), rz.RAZER_F32, ctypes.byref(s), FAKE_WS, 4096, None) == rz.RAZER_E_INVALID
    assert L.razer_quantize_weight(FAKE_X, rz.RAZER_F32, ctypes.byref(s), FAKE_WS, 16, None) == rz.RAZER_E_INVALID
    assert L.razer_quantize_weight(FAKE_X, rz.RAZER_F32, ctypes.byref(s), None, 4096, None) == rz.RAZER_E_INVALID
    assert L.razer_quantize_weight(FAKE_X, 9, ctypes.byref(s), FAKE_WS, 4096, None) == rz.RAZER_E_INVALID
    assert L.razer_quantize_weight(FAKE_X, rz.RAZER_F32, None, FAKE_WS, 4096, None) == rz.RAZER_E_INVALID
    a = _packed(kind=rz.RAZER_ACT, off=(-2, 99))  # act kind ignores the second offset ...
    a.sv_off_half[0] = -9                          # ... but checks the first
    assert L.razer_quantize_act(FAKE_X, rz.RAZER_BF16, ctypes.byref(a), FAKE_WS, 4096, None) == rz.RAZER_E_INVALID


def test_products_reject_bad_arguments():
    L = rz.lib()
    s = _packed()
    y = ctypes.c_void_p(0x6000)
    assert L.razer_gemv(FAKE_X, rz.RAZER_F32, ctypes.byref(s), y, rz.RAZER_F32, None, 0, None) == rz.RAZER_E_UNSUPPORTED
    assert L.razer_gemv(FAKE_X, 7, ctypes.byref(s), y, rz.RAZER_F32, None, 0, None) == rz.RAZER_E_INVALID
    assert L.razer_gemv(FAKE_X, rz.RAZER_F16, ctypes.byref(s), None, rz.RAZER_F32, None, 0, None) == rz.RAZER_E_INVALID
    assert L.razer_gemv(ctypes.c_void_p(0x4002), rz.RAZER_F16, ctypes.byref(s), y, rz.RAZER_F32, None, 0, None) == rz.RAZER_E_INVALID
    big = _packed(cols=65536 + 16)
    assert L.razer_gemv(FAKE_X, rz.RAZER_F16, ctypes.byref(big), y, rz.RAZER_F32, None, 0, None) == rz.RAZER_E_UNSUPPORTED
    assert L.razer_gemm(FAKE_X, rz.RAZER_BF16, -1, ctypes.byref(s), y, rz.RAZER_F32, None, 0, None) == rz.RAZER_E_INVALID
    assert L.razer_gemm(FAKE_X, rz.RAZER_BF16, 0, ctypes.byref(s), y, rz.RAZER_F32, None, 0, None) == rz.RAZER_OK
    assert L.razer_gemm(FAKE_X, rz.RAZER_F32, 4, ctypes.byref(s), y, rz.RAZER_F32, None, 0, None) == rz.RAZER_E_UNSUPPORTED
    assert L.razer_gemm(FAKE_X, rz.RAZER_BF16, 4, ctypes.byref(s), ctypes.c_void_p(0x6004), rz.RAZER_F32, None, 0, None) == rz.RAZER_E_INVALID
    bad = _packed(cols=20)
    assert L.razer_dequant(ctypes.byref(bad), y, rz.RAZER_F32, None) == rz.RAZER_E_INVALID
    assert L.razer_dequant(ctypes.byref(s), y, 5, None) == rz.RAZER_E_INVALID
    assert L.razer_dequant(ctypes.byref(s), None, rz.RAZER_F32, None) == rz.RAZER_E_INVALID


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(rz, "_lib", None)
    monkeypatch.setattr(rz, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        rz.lib()


@pytest.mark.parametrize("args", [
    dict(cols=24),                 # cols % 16 != 0
    dict(rows=-1),
    dict(off0=8),                  # offset outside [-7, 7]
    dict(off0=-8),
    dict(dt=7),                    # unknown dtype
    dict(sse=None),
    dict(sse=0x6004),              # misaligned sse
    dict(w=None),
    dict(w=0x4008),                # misaligned weight
    dict(ws=None),
    dict(wsb=16),                  # workspace too small
])
def test_offset_search_rejects_bad_arguments(args):
    a = dict(w=0x4000, dt=rz.RAZER_F32, rows=4, cols=32, off0=-2, sse=0x6000, ws=0x5000, wsb=1 << 20)
    a.update(args)
    st = rz.lib().razer_weight_offset_sse(ctypes.c_void_p(a["w"]), a["dt"], a["rows"], a["cols"], a["off0"],
                                          ctypes.c_void_p(a["sse"]), ctypes.c_void_p(a["ws"]), a["wsb"], None)
    assert st == rz.RAZER_E_INVALID


def test_offset_search_workspace_covers_partials():
    # amax partials plus 15 fp64 sums per workgroup
    assert rz.razer_workspace_bytes(rz.RAZER_OP_OFFSET_SEARCH, 0, 28672, 8192) >= 4096 + 15 * 8
    assert rz.razer_workspace_bytes(rz.RAZER_OP_OFFSET_SEARCH, 0, 1, 16) >= 4096 + 15 * 8


@pytest.mark.parametrize("case", ["cols_differ", "bad_x", "bad_w", "y_null", "y_misaligned", "ws_small",
                                  "ws_misaligned", "dtype"])
def test_gemm_w4a4_rejects_bad_arguments(case):
    x = _packed(kind=rz.RAZER_ACT, rows=2, cols=32, off=(-2, -2))
    w = _packed(rows=8, cols=32)
    y, ws, wsb, dt = 0x7000, 0x10000, 1 << 20, rz.RAZER_BF16
    if case == "cols_differ":
        w.cols = 48
    elif case == "bad_x":
        x.cols = 24
    elif case == "bad_w":
        w.sv_off_half[1] = 9
    elif case == "y_null":
        y = 0
    elif case == "y_misaligned":
        y = 0x7004
    elif case == "ws_small":
        wsb = 16
    elif case == "ws_misaligned":
        ws = 0x10010
    elif case == "dtype":
        dt = 9
    st = rz.lib().razer_gemm_w4a4(ctypes.byref(x), ctypes.byref(w), ctypes.c_void_p(y), dt,
                                  ctypes.c_void_p(ws), wsb, None)
    assert st == rz.RAZER_E_INVALID


def test_gemm_w4a4_workspace_holds_both_intermediates():
    m, n, k = 7, 40, 96
    assert rz.razer_workspace_bytes(rz.RAZER_OP_GEMM_W4A4, m, n, k) >= m * k * 2 + m * n * 4
    assert rz.razer_workspace_bytes(rz.RAZER_OP_GEMM_W4A4, 0, n, k) == 0


def _group_call(ws, ys, count=None, x=FAKE_X, x_dt=rz.RAZER_F16, y_dt=rz.RAZER_F16):
    P = ctypes.POINTER(rz.razer_packed)
    arr = (P * max(1, len(ws)))(*[ctypes.pointer(s) for s in ws])
    yarr = (ctypes.c_void_p * max(1, len(ys)))(*ys)
    n = len(ws) if count is None else count
    return rz.lib().razer_gemv_group(x, x_dt, arr, yarr, n, y_dt, None)


@pytest.mark.parametrize("case", ["count0", "count5", "unequal_k", "bad_packed", "null_y", "misaligned_y",
                                  "null_x", "bad_dtype"])
def test_gemv_group_rejects_bad_arguments(case):
    a, b = _packed(rows=8, cols=64), _packed(rows=4, cols=64)
    ws, ys, kw = [a, b], [0x6000, 0x7000], {}
    if case == "count0":
        kw["count"] = 0
    elif case == "count5":
        ws, ys = [a] * 5, [0x6000] * 5
    elif case == "unequal_k":
        b.cols = 80
    elif case == "bad_packed":
        b.sv_off_half[0] = 9
    elif case == "null_y":
        ys = [0x6000, 0]
    elif case == "misaligned_y":
        ys = [0x6008, 0x7000]
    elif case == "null_x":
        kw["x"] = None
    elif case == "bad_dtype":
        kw["y_dt"] = 7
    assert _group_call(ws, ys, **kw) == rz.RAZER_E_INVALID


def test_gemv_group_unsupported_like_gemv():
    a = _packed(rows=8, cols=64)
    assert _group_call([a], [0x6000], x_dt=rz.RAZER_F32) == rz.RAZER_E_UNSUPPORTED
    big = _packed(rows=8, cols=65536 + 16)
    assert _group_call([big], [0x6000]) == rz.RAZER_E_UNSUPPORTED


def test_layout_variants_host_checks():
    L = rz.lib()
    a = _packed(kind=rz.RAZER_ACT, off=(-2, 0), cols=128)
    a.scale_fmt = rz.RAZER_SCALE_F16  # FP16 group scales are for weights only
    assert L.razer_quantize_act(FAKE_X, rz.RAZER_BF16, ctypes.byref(a), FAKE_WS, 4096, None) == rz.RAZER_E_INVALID
    # the products take 16-element blocks with byte scales; the GEMV calls and
    # razer_gemm also take 128-element blocks with FP16 scales (not checked here:
    # that would launch), razer_gemm_w4a4 does not
    y = ctypes.c_void_p(0x6000)
    x = _packed(kind=rz.RAZER_ACT, off=(-2, 0), rows=2, cols=128)
    for blog2, fmt in ((5, 0), (7, 0), (4, 1), (7, 1)):
        w = _packed(rows=8, cols=128)
        w.block_log2, w.scale_fmt = blog2, fmt
        if (blog2, fmt) != (7, 1):
            assert L.razer_gemv(FAKE_X, rz.RAZER_F16, ctypes.byref(w), y, rz.RAZER_F16, None, 0, None) == rz.RAZER_E_UNSUPPORTED
            assert _group_call([w], [0x6000]) == rz.RAZER_E_UNSUPPORTED
            assert L.razer_gemm(FAKE_X, rz.RAZER_F16, 4, ctypes.byref(w), y, rz.RAZER_F16, FAKE_WS, 1 << 20,
                                None) == rz.RAZER_E_UNSUPPORTED
        assert L.razer_gemm_w4a4(ctypes.byref(x), ctypes.byref(w), y, rz.RAZER_BF16, FAKE_WS, 1 << 20, None) == rz.RAZER_E_UNSUPPORTED
    # one layout per grouped launch
    g128 = _packed(rows=8, cols=128)
    g128.block_log2, g128.scale_fmt = 7, 1
    assert _group_call([_packed(rows=8, cols=128), g128], [0x6000, 0x7000]) == rz.RAZER_E_UNSUPPORTED


def test_gemm_rejects_a_workspace_smaller_than_its_k_split():
    # M = 16 on a 28672 x 8192 weight splits K across workgroups, whose fp32
    # partial sums need a workspace; a smaller or missing one is refused on the
    # host before anything is enqueued.
    L = rz.lib()
    need = rz.razer_workspace_bytes(rz.RAZER_OP_GEMM, 16, 28672, 8192)
    assert need >= 2 * 16 * 28672 * 4
    w = _packed(rows=28672, cols=8192)
    y = ctypes.c_void_p(0x6000)
    for ws, nbytes in ((None, need), (FAKE_WS, need - 4), (FAKE_WS, 256)):
        assert L.razer_gemm(FAKE_X, rz.RAZER_BF16, 16, ctypes.byref(w), y, rz.RAZER_BF16, ws, nbytes,
                            None) == rz.RAZER_E_INVALID
