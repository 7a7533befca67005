#!/usr/bin/env python3
"""Benchmark of the RaZeR-NVFP4 W4A16 layer on one MI355X.

Headline (the JSON line's ``value``): batch-1 decode throughput of the
Llama-3-8B-shaped linear layers -- qkv [6144,4096], gate [14336,4096],
up [14336,4096], down [4096,14336] -- with fp16 activations and RaZeR-W4
weights (0.02 * Student-t(5)), over L distinct layer copies (default 8, 906 MB
of packed weights, larger than the 256 MB Infinity Cache).  One step = one
token through the L layers = 3L launches replayed from a HIP graph: razer_gemv
for qkv and down, razer_gemv_group for gate and up (the two read the same x);
--per-matrix times 4L razer_gemv launches instead (also reported as a row).
``value`` is algorithmic GB/s (packed weights + x + y + tensor scale, each
counted once) over the timed steps.  Every timed region, the headline's and
each row's, follows W warmup replays and then at least SETTLE_MS (100 ms) of
untimed replays, so that the clocks have left their idle state (the JSON line
gives the number of settling steps); the K timed steps are whole steps.

Also measured in the same run (the ``rows`` object): the weight and activation
encoders (Gelem/s, GB/s, special-value-search overhead), the small-batch GEMM
sweep (M = 1..32, GB/s) and the M=2048 prefill GEMM (TFLOP/s), each on its own
synthetic workload, with two practical ceilings beside them: a plain device copy
at the decode launch sizes and the library's dense bf16 GEMM at the prefill
shape; ``roofline`` for the GEMV kernel; ``cpu_baseline`` = the CPU oracle over
one decode step (single thread, about 14 s).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L]
                       [--no-rows] [--no-cpu-baseline] [--eager] [--per-matrix]
       python bench.py --counters {prefill,w4a4,quantize_weight,quantize_act,dequant,small_batch}
       python bench.py --copy-calibration
       python bench.py --traffic-summary RD.csv WR.csv FS.csv CAL_RD.csv CAL_WR.csv CAL_FS.csv

--eager replays the decode launches without a graph (for counter passes);
--counters W runs one row's launches (prefill, w4a4, quantize_weight,
quantize_act, dequant, small_batch) three times, untimed, for counter passes;
--copy-calibration runs a plain elementwise copy (negation) of 512 MiB, the check
that the request counters are byte-exact; --traffic-summary turns six rocprofv3
counter CSVs (decode launches: TCC_EA0_RDREQ_{32B,64B,128B}_sum, TCC_EA0_WRREQ{,_64B}_sum,
FETCH_SIZE; the same three for the copy) into profiles/traffic.json, stamped with
the hash of the GEMV sources.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
METRIC = "RaZeR W4A16 GEMV/GEMM GB/s & TFLOP/s (% roofline); quantizer Gelem/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def packed_bytes(n, k, block=16, scale_bytes=1):
    return n * k // 2 + n * k // block * scale_bytes + 4


def gemv_bytes(n, k, xb=2, yb=2):
    return packed_bytes(n, k) + k * xb + n * yb


def clone_packed(rz, p):
    q = rz.PackedTensor(p.kind, p.rows, p.cols, p.offsets, p.codes.device, p.flags, p.block,
                        p.scale_fmt)
    q.codes.copy_(p.codes)
    q.scales.copy_(p.scales)
    q.tensor_scale.copy_(p.tensor_scale)
    return q


# Untimed work before every timed region.  After an idle spell the clocks take
# tens of milliseconds to settle: the decode step replayed right after a one
# second pause runs 250-290 us per step for its first ten steps and settles at
# about 226 us after some hundred (about 25 ms); the prefill GEMM dips to
# 820-870 TFLOP/s before it climbs to about 1080 over some 40 ms.  Timing only
# steady-state replays keeps those transients out of every figure.
SETTLE_MS = 100.0


def settle(torch, run, min_ms=SETTLE_MS, chunk=8):
    """Call run() (untimed) in chunks until at least min_ms of wall time have
    passed, then synchronize; returns the number of calls."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for _ in range(chunk):
            run()
        n += chunk
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= min_ms:
            return n


class GraphTimer:
    """Capture fn() (a batch of launches on the current stream) in a HIP graph
    and time replays with events on that stream, after warmup replays and
    SETTLE_MS of untimed ones."""

    def __init__(self, torch, fn, warmup=2):
        self.torch = torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(warmup):
                fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            fn()
        torch.cuda.synchronize()

    def time(self, iters, warmup=1, settle_ms=SETTLE_MS):
        t = self.torch
        for _ in range(warmup):
            self.g.replay()
        t.cuda.synchronize()
        if settle_ms > 0:
            settle(t, self.g.replay, settle_ms)
        st = t.cuda.current_stream()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(iters):
            self.g.replay()
        e1.record(st)
        e1.synchronize()
        return e0.elapsed_time(e1) / iters  # ms per replay


def source_hash(*names):
    h = hashlib.sha1()
    for n in names:
        h.update(open(os.path.join(ROOT, "nvfp4_razer_w4a16_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


COPY_BYTES = 512 << 20  # the calibration copy reads and writes this many bytes
# razer_gemv runs gemv_kernel for more than 4096 rows and smallm_kernel up to 4096
DECODE_KERNELS = ("gemv_kernel", "smallm_kernel")
DECODE_SOURCES = ("rz_gemv.hip", "rz_smallm.hip", "rz_device.h")


COUNTER_WORKLOADS = ("prefill", "w4a4", "quantize_weight", "quantize_act", "dequant", "small_batch")


def run_counter_workload(torch, rz, synth, name):
    """The launches of one row's workload, three times each, eager and untimed,
    so that counter passes see only those kernels (plus input setup)."""
    dev = torch.device("cuda:0")
    if name in ("prefill", "w4a4", "quantize_weight", "dequant"):
        w = torch.from_numpy(synth.prefill_weight()).to(dev)
        wp = rz.razer_quantize_weight(w, (-2, 4))
    if name == "quantize_weight":
        ws = torch.empty(rz.razer_workspace_bytes(rz.RAZER_OP_QUANTIZE_WEIGHT, 28672, 0, 8192),
                         dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(3):
            rz.razer_quantize_weight(w, out=wp, workspace=ws)
    elif name == "quantize_act":
        x = synth.act_quant_x().to(dev)
        out = rz.PackedTensor(rz.RAZER_ACT, 4096, 8192, (-2,), dev)
        ws = torch.empty(rz.razer_workspace_bytes(rz.RAZER_OP_QUANTIZE_ACT, 4096, 0, 8192),
                         dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(3):
            rz.razer_quantize_act(x, out=out, workspace=ws)
    elif name == "prefill":
        x = synth.prefill_x().to(dev)
        y = torch.empty((2048, 28672), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        for _ in range(3):
            rz.razer_gemm(x, wp, out=y)
    elif name == "w4a4":
        xq = rz.razer_quantize_act(synth.prefill_x().to(dev))
        y = torch.empty((2048, 28672), dtype=torch.bfloat16, device=dev)
        w4 = torch.empty(rz.razer_workspace_bytes(rz.RAZER_OP_GEMM_W4A4, 2048, 28672, 8192),
                         dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(3):
            rz.razer_gemm_w4a4(xq, wp, out=y, workspace=w4)
    elif name == "small_batch":
        for n, k in ((28672, 8192), (4096, 4096)):
            wsb = rz.razer_quantize_weight(torch.from_numpy(synth.small_batch_weight(n, k)).to(dev), (-2, 4))
            for m in (4, 8, 16, 32):
                x = synth.small_batch_x(m, k).to(dev)
                y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
                ws = torch.empty(max(1, rz.razer_workspace_bytes(rz.RAZER_OP_GEMM, m, n, k)),
                                 dtype=torch.uint8, device=dev)
                torch.cuda.synchronize()
                for _ in range(3):
                    rz.razer_gemm(x, wsb, out=y, workspace=ws)
            del wsb
    elif name == "dequant":
        out = torch.empty((28672, 8192), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        for _ in range(3):
            rz.razer_dequant(wp, out=out)
    torch.cuda.synchronize()
    log(f"counters: {name} x3 done")


def copy_calibration():
    import torch

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):  # one elementwise kernel: reads and writes COPY_BYTES each
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: 5 elementwise copies of {COPY_BYTES} bytes")


def _counters_per_dispatch(path, name_parts):
    """{dispatch id: {counter: value summed over its instances}} for the
    dispatches of kernels whose names contain one of name_parts, from a
    rocprofv3 counter_collection CSV, plus each dispatch's kernel name and grid."""
    import csv
    from collections import defaultdict

    per = defaultdict(lambda: defaultdict(float))
    what = {}
    for r in csv.DictReader(open(path)):
        if any(p in r["Kernel_Name"] for p in name_parts):
            per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            what[r["Dispatch_Id"]] = (r["Kernel_Name"], int(r["Grid_Size"]))
    if not per:
        raise SystemExit(f"no dispatch of {name_parts!r} in {path}")
    return per, what


def _read_bytes(c):
    return 32 * c["TCC_EA0_RDREQ_32B_sum"] + 64 * c["TCC_EA0_RDREQ_64B_sum"] + 128 * c["TCC_EA0_RDREQ_128B_sum"]


def _write_bytes(c):
    return 32 * (c["TCC_EA0_WRREQ_sum"] - c["TCC_EA0_WRREQ_64B_sum"]) + 64 * c["TCC_EA0_WRREQ_64B_sum"]


def traffic_summary(rd_csv, wr_csv, fs_csv, cal_rd_csv, cal_wr_csv, cal_fs_csv):
    """HBM bytes per decode launch from the L2-to-memory request counters:
    reads = 32 n32 + 64 n64 + 128 n128 (TCC_EA0_RDREQ_{32B,64B,128B}, summed
    over the L2 channels), writes = 32 n32 + 64 n64 (TCC_EA0_WRREQ, _64B).
    The calibration copy (COPY_BYTES read and written) checks that these
    counts are byte-exact.  FETCH_SIZE, scaled by what it reads for the same
    copy, is kept beside them as a cross-check."""
    rd, what = _counters_per_dispatch(rd_csv, DECODE_KERNELS)
    wr, _ = _counters_per_dispatch(wr_csv, DECODE_KERNELS)
    fs, _ = _counters_per_dispatch(fs_csv, DECODE_KERNELS)
    crd, _ = _counters_per_dispatch(cal_rd_csv, ("elementwise",))
    cwr, _ = _counters_per_dispatch(cal_wr_csv, ("elementwise",))
    cfs, _ = _counters_per_dispatch(cal_fs_csv, ("elementwise",))
    big = lambda d, f: max(f(c) for c in d.values())  # the copy dispatch (others are tiny fills)
    cal_read, cal_write = big(crd, _read_bytes), big(cwr, _write_bytes)
    fs_scale = COPY_BYTES / (big(cfs, lambda c: c["FETCH_SIZE"]) * 1024.0)
    classes = {}
    for d, (name, grid) in what.items():
        key = f"{'smallm_kernel' if 'smallm' in name else 'gemv_kernel'} grid {grid}"
        cl = classes.setdefault(key, {"read": [], "write": [], "fetch_size_scaled": []})
        cl["read"].append(_read_bytes(rd[d]))
        if d in wr:
            cl["write"].append(_write_bytes(wr[d]))
    for d, (name, grid) in _counters_per_dispatch(fs_csv, DECODE_KERNELS)[1].items():
        key = f"{'smallm_kernel' if 'smallm' in name else 'gemv_kernel'} grid {grid}"
        classes[key]["fetch_size_scaled"].append(fs[d]["FETCH_SIZE"] * 1024.0 * fs_scale)
    mean = lambda v: sum(v) / len(v) if v else None
    per_class = {k: {"read_bytes": mean(v["read"]), "write_bytes": mean(v["write"]),
                     "fetch_size_scaled_bytes": mean(v["fetch_size_scaled"]), "dispatches": len(v["read"])}
                 for k, v in sorted(classes.items())}
    n = len(per_class)
    total = sum(v["read_bytes"] + v["write_bytes"] for v in per_class.values()) / n
    src = source_hash(*DECODE_SOURCES)
    out = {"gemv_decode": {
        "source_hash": src, "bytes_per_launch": round(total),
        "method": "TCC_EA0_RDREQ_{32B,64B,128B} and TCC_EA0_WRREQ{,_64B} request counts x request size",
        "per_launch_class": per_class,
        "copy_check": {"read_bytes": cal_read, "write_bytes": cal_write, "copy_bytes": COPY_BYTES,
                       "fetch_size_scale": fs_scale}}}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    json.dump(out, open(path, "w"), indent=1)
    print(json.dumps(out))


def load_traffic(kernel_key, src_hash):
    """HBM traffic measured by rocprofv3 counters for the current kernel source,
    or None when the counters are missing or were taken on another version."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        d = json.load(open(path))[kernel_key]
    except Exception:
        return None
    if d.get("source_hash") != src_hash:
        return None
    return d.get("bytes_per_launch")


# ---- headline: decode GEMV -----------------------------------------------------

def setup_decode(torch, rz, synth, layers, block=16, scale_fmt=0):
    """Decode step launches over `layers` copies of the layer's weights: grouped
    (qkv; gate and up in one launch, they read the same x; down) and per matrix.
    block / scale_fmt: the weights' layout (default: 16-element blocks, byte scales)."""
    dev = torch.device("cuda:0")
    names = ["qkv", "gate", "up", "down"]
    base = {}
    for name in names:
        w = torch.from_numpy(synth.llama3_8b_decode_weight(name)).to(dev)
        base[name] = rz.razer_quantize_weight(w, (-2, 4), block=block, scale_fmt=scale_fmt)
        del w
    torch.cuda.synchronize()
    mats = [{n: (base[n] if li == 0 else clone_packed(rz, base[n])) for n in names}
            for li in range(layers)]
    xs = {4096: synth.llama3_8b_decode_x(4096).to(dev).reshape(-1),
          14336: synth.llama3_8b_decode_x(14336).to(dev).reshape(-1)}
    ys = {n: torch.empty(base[n].rows, dtype=torch.float16, device=dev) for n in names}
    out = {}
    for kind, groups in (("grouped", [("qkv",), ("gate", "up"), ("down",)]),
                         ("per_matrix", [(n,) for n in names])):
        launches = [(xs[layer[g[0]].cols], [layer[n] for n in g], [ys[n] for n in g])
                    for layer in mats for g in groups]
        # algorithmic bytes: packed weights, x once per launch, y
        sbytes = 2 if scale_fmt else 1
        step_bytes = sum(sum(packed_bytes(m.rows, m.cols, block, sbytes) + 2 * m.rows for m in ws)
                         + 2 * ws[0].cols for _, ws, _ in launches)
        out[kind] = (launches, step_bytes)
    return out, base


def run_launches(rz, launches):
    for x, ws, ys in launches:
        if len(ws) == 1:
            rz.razer_gemv(x, ws[0], out=ys[0])
        else:
            rz.razer_gemv_group(x, ws, outs=ys)


def launch_bytes(launch):
    """Algorithmic bytes of one decode launch: packed weights, y, x once."""
    _, ws, _ = launch
    return sum(packed_bytes(m.rows, m.cols, m.block, 2 if m.scale_fmt else 1) + 2 * m.rows for m in ws) \
        + 2 * ws[0].cols


DECODE_CLASSES = ("qkv", "gate_up", "down")  # the grouped step's launches, in order per layer


def per_kernel_rates(torch, rz, launches, steps):
    """Each launch class of the grouped decode step (qkv: gemv_kernel; gate and
    up: one gemv_kernel launch; down: smallm_kernel) timed on its own: the
    class's launches over the layer copies in one HIP graph, HIP events on the
    launch stream; average duration per launch and the GB/s it implies."""
    out = {}
    for ci, name in enumerate(DECODE_CLASSES):
        ls = launches[ci::len(DECODE_CLASSES)]
        ms = GraphTimer(torch, lambda: run_launches(rz, ls), warmup=1).time(steps) / len(ls)
        b = launch_bytes(ls[0])
        out[name] = {"avg_launch_us": round(ms * 1e3, 3), "algorithmic_bytes": b,
                     "achieved_gbs": round(b / ms / 1e6, 1), "frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4)}
    return out


def ceiling_lib():
    """libceiling.so: the plain-read and register-only MFMA probes (bench only)."""
    import ctypes

    L = ctypes.CDLL(os.path.join(ROOT, "nvfp4_razer_w4a16_amd", "libceiling.so"))
    L.rzc_read.restype = ctypes.c_int
    L.rzc_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.rzc_mfma_loop.restype = ctypes.c_int
    L.rzc_mfma_loop.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.rzc_read_tiles.restype = ctypes.c_int
    L.rzc_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_void_p]
    return L


def tile_read_floor(torch, mats, cus, steps=5):
    """Plain read of each packed weight in mats with the load pattern and grid
    of the small-batch streaming kernel (nothing computed), us per weight."""
    L = ceiling_lib()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def run():
        st = torch.cuda.current_stream().cuda_stream
        for mm in mats:
            if L.rzc_read_tiles(mm.codes.data_ptr(), mm.scales.data_ptr(), mm.rows, mm.cols, cus,
                                sink.data_ptr(), st) != 0:
                raise RuntimeError("rzc_read_tiles failed")

    return GraphTimer(torch, run, warmup=1).time(steps) / len(mats) * 1e3


def step_read_floor(torch, launches, step_bytes, steps):
    """The decode step's plain-read floor: for every GEMV launch of the step,
    one launch that only reads the same weight bytes (codes and scales of each
    weight in it), 16 KiB per 256-thread workgroup in 16-byte non-temporal
    loads, in the step's order, replayed from a HIP graph like the step itself."""
    import ctypes

    L = ceiling_lib()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    prepared = []
    for _, ws, _ in launches:
        bufs = [t for w in ws for t in (w.codes, w.scales)]
        prepared.append(((ctypes.c_void_p * len(bufs))(*[b.data_ptr() for b in bufs]),
                         (ctypes.c_int64 * len(bufs))(*[b.numel() for b in bufs]), len(bufs)))

    def run():
        st = torch.cuda.current_stream().cuda_stream
        for ptrs, ns, c in prepared:
            if L.rzc_read(ptrs, ns, c, sink.data_ptr(), st) != 0:
                raise RuntimeError("rzc_read failed")

    ms = GraphTimer(torch, run, warmup=1).time(steps)
    return {"workload": "plain read of the decode step's weight bytes, one read launch per GEMV launch "
                        f"({len(launches)} per step), 16 KiB per workgroup, HIP graph",
            "us_per_step": ms * 1e3, "gbs_on_step_bytes": step_bytes / ms / 1e6,
            "frac_hbm": step_bytes / ms / 1e6 / HBM_PEAK_GBS}


def mfma_loop_ceiling(torch, cus, reps=5, iters=20000):
    """Register-only v_mfma_f32_32x32x16_bf16 loop: random bf16 operands, two
    waves per SIMD on every CU (the prefill product's layout), no memory
    traffic; TFLOP/s from HIP events."""
    L = ceiling_lib()
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    wgs = 2 * cus
    st = torch.cuda.current_stream()
    for _ in range(2):
        L.rzc_mfma_loop(iters // 4, wgs, sink.data_ptr(), st.cuda_stream)
    torch.cuda.synchronize()
    settle(torch, lambda: L.rzc_mfma_loop(iters // 4, wgs, sink.data_ptr(), st.cuda_stream))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        if L.rzc_mfma_loop(iters, wgs, sink.data_ptr(), st.cuda_stream) != 0:
            raise RuntimeError("rzc_mfma_loop failed")
    e1.record(st)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = wgs * 4 * iters * 2 * (2.0 * 32 * 32 * 16)
    return {"workload": f"v_mfma_f32_32x32x16_bf16 on register operands (random bf16), {wgs} workgroups of "
                        "4 waves (2 waves per SIMD), no memory traffic",
            "ms": ms, "tflops": flops / ms / 1e9, "frac_mfma": flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS}


# ---- other rows --------------------------------------------------------------------

def rel_sse(torch, rz, x, packed):
    """sum (x - dequant(packed))^2 / sum x^2, in fp64 (a quality figure, not timed)."""
    d = rz.razer_dequant(packed, torch.float32)
    e = float(torch.sum((x.float() - d).double().square()))
    del d
    return e / float(torch.sum(x.double().square()))


def hbm_copy_floor(torch, dev):
    """Context for the GEMV's roofline fraction: a plain device-to-device copy
    (torch's copy kernel, graph-replayed like the decode step) at the sizes one
    decode launch moves, and at 512 MiB.  GB/s counts bytes read + written."""
    out = {}
    for mb in (14, 33, 66, 512):
        nbytes = mb * (1 << 20)
        copies = max(1, int(1024e6 // nbytes))  # cycle through > 1 GB so reads come from HBM
        src = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
        dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        t = GraphTimer(torch, lambda: [dst.copy_(sv) for sv in src])
        ms = t.time(10) / copies
        out[f"{mb}MiB"] = {"us": ms * 1e3, "gbs": 2 * nbytes / ms / 1e6,
                           "frac_hbm": 2 * nbytes / ms / 1e6 / HBM_PEAK_GBS}
        del src, dst, t
    torch.cuda.empty_cache()
    return out


def bench_rows(torch, rz, synth, args, decode_base):
    dev = torch.device("cuda:0")
    rows = {"hbm_copy_floor": hbm_copy_floor(torch, dev)}

    # weight encoder on the decode layer's weights (offline path, 4 candidates)
    ws = {}
    for name in ("gate", "down"):
        w = torch.from_numpy(synth.llama3_8b_decode_weight(name)).to(dev)
        out = rz.PackedTensor(rz.RAZER_WEIGHT, w.shape[0], w.shape[1], (-2, 4), dev)
        out0 = rz.PackedTensor(rz.RAZER_WEIGHT, w.shape[0], w.shape[1], (-2, 4), dev,
                               rz.RAZER_FLAG_NO_REMAP)
        ws[name] = (w, out, out0)
    n_el = sum(w.numel() for w, _, _ in ws.values())
    t = GraphTimer(torch, lambda: [rz.razer_quantize_weight(w, out=o) for w, o, _ in ws.values()])
    ms = t.time(20)
    t0 = GraphTimer(torch, lambda: [rz.razer_quantize_weight(w, out=o0) for w, _, o0 in ws.values()])
    ms0 = t0.time(20)
    rows["quantize_weight"] = {
        "workload": "gate [14336,4096] + down [4096,14336] fp32, 0.02*t(5), offsets (-2,4)",
        "gelem_per_s": n_el / ms / 1e6, "ms": ms,
        "gbs_1read": n_el * (4 + 0.5625) / ms / 1e6,
        "frac_hbm_1read": n_el * (4 + 0.5625) / ms / 1e6 / HBM_PEAK_GBS,
        "no_remap_ms": ms0, "search_overhead_pct": 100.0 * (ms - ms0) / ms0}
    del ws, t, t0
    torch.cuda.empty_cache()

    # activation encoder X[4096, 8192] bf16 (online path, 2 candidates), over
    # 8 distinct copies of X and of the output (690 MB in all, well above the
    # 256 MB Infinity Cache), so every read of X comes from HBM
    x0 = synth.act_quant_x().to(dev)
    ncopy = 8
    xs_ = [x0] + [x0.clone() for _ in range(ncopy - 1)]
    outs = [rz.PackedTensor(rz.RAZER_ACT, 4096, 8192, (-2,), dev) for _ in range(ncopy)]
    outs0 = [rz.PackedTensor(rz.RAZER_ACT, 4096, 8192, (-2,), dev, rz.RAZER_FLAG_NO_REMAP) for _ in range(ncopy)]
    wsp = torch.empty(rz.razer_workspace_bytes(rz.RAZER_OP_QUANTIZE_ACT, 4096, 0, 8192),
                      dtype=torch.uint8, device=dev)
    t = GraphTimer(torch, lambda: [rz.razer_quantize_act(xi, out=o, workspace=wsp) for xi, o in zip(xs_, outs)])
    ms = t.time(10) / ncopy
    t0 = GraphTimer(torch, lambda: [rz.razer_quantize_act(xi, out=o, workspace=wsp) for xi, o in zip(xs_, outs0)])
    ms0 = t0.time(10) / ncopy
    n_el = x0.numel()
    rows["quantize_act"] = {
        "workload": "X [4096,8192] bf16 N(0,1), 16 channels x50, 1% tokens x5; 8 distinct copies of X and "
                    "of the packed output cycled (X read from HBM)",
        "gelem_per_s": n_el / ms / 1e6, "ms": ms,
        "gbs_1read": n_el * (2 + 0.5625) / ms / 1e6,
        "frac_hbm_1read": n_el * (2 + 0.5625) / ms / 1e6 / HBM_PEAK_GBS,
        "gbs_2pass": n_el * (2 * 2 + 0.5625) / ms / 1e6,
        "no_remap_ms": ms0, "search_overhead_pct": 100.0 * (ms - ms0) / ms0}
    del x0, xs_, outs, outs0, t, t0
    torch.cuda.empty_cache()

    # small-batch GEMM sweep
    sweep = {}
    for (n, k) in synth.SMALL_BATCH_SHAPES:
        w = torch.from_numpy(synth.small_batch_weight(n, k)).to(dev)
        base = rz.razer_quantize_weight(w, (-2, 4))
        del w
        copies = max(1, int(640e6 // packed_bytes(n, k)))  # > 2x the Infinity Cache
        mats = [base] + [clone_packed(rz, base) for _ in range(copies - 1)]
        floor_us = tile_read_floor(torch, mats, torch.cuda.get_device_properties(0).multi_processor_count)
        sweep[f"{n}x{k}_tile_read_floor"] = {
            "workload": "plain read of the packed weight with the streaming kernel's loads and grid",
            "us": floor_us, "gbs": packed_bytes(n, k) / floor_us / 1e3,
            "frac_hbm": packed_bytes(n, k) / floor_us / 1e3 / HBM_PEAK_GBS}
        for m in synth.SMALL_BATCH_M:
            x = synth.small_batch_x(m, k).to(dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            wsb = max(1, rz.razer_workspace_bytes(rz.RAZER_OP_GEMM, m, n, k))
            wsp = torch.empty(wsb, dtype=torch.uint8, device=dev)
            t = GraphTimer(torch, lambda: [rz.razer_gemm(x, mm, out=y, workspace=wsp) for mm in mats])
            ms = t.time(5) / len(mats)
            byts = packed_bytes(n, k) + m * k * 2 + m * n * 2
            # the same launches with the untrimmed plan (every CU, the most K splits)
            umats = [mm.with_flags(rz.RAZER_FLAG_UNTRIMMED_PLAN) for mm in mats]
            wsu = torch.empty(max(1, rz.razer_workspace_bytes(rz.RAZER_OP_GEMM_UNTRIMMED, m, n, k)),
                              dtype=torch.uint8, device=dev)
            tu = GraphTimer(torch, lambda: [rz.razer_gemm(x, mm, out=y, workspace=wsu) for mm in umats])
            ms_u = tu.time(5) / len(mats)
            sweep[f"{n}x{k}_m{m}"] = {"us": ms * 1e3, "gbs": byts / ms / 1e6,
                                      "frac_hbm": byts / ms / 1e6 / HBM_PEAK_GBS,
                                      "tflops": 2.0 * m * n * k / ms / 1e9,
                                      "untrimmed_us": ms_u * 1e3,
                                      "plan_gain_pct": 100.0 * (ms_u - ms) / ms_u,
                                      "frac_of_tile_read_floor": floor_us / (ms * 1e3)}
            del t, tu, umats, wsu
        del mats, base
        torch.cuda.empty_cache()
    rows["gemm_small_batch"] = sweep

    # the same sweep on the pages' kernel layout (128-element blocks, FP16
    # scales with the metadata in the sign and top exponent bits), 28672 x 8192
    n, k = 28672, 8192
    w = torch.from_numpy(synth.small_batch_weight(n, k)).to(dev)
    base = rz.razer_quantize_weight(w, (-2, 4), block=128, scale_fmt=rz.RAZER_SCALE_F16)
    del w
    pbytes = packed_bytes(n, k, 128, 2)
    mats = [base] + [clone_packed(rz, base) for _ in range(max(1, int(640e6 // pbytes)) - 1)]
    sweep = {}
    for m in synth.SMALL_BATCH_M:
        x = synth.small_batch_x(m, k).to(dev)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        wsp = torch.empty(max(1, rz.razer_workspace_bytes(rz.RAZER_OP_GEMM, m, n, k)), dtype=torch.uint8,
                          device=dev)
        t = GraphTimer(torch, lambda: [rz.razer_gemm(x, mm, out=y, workspace=wsp) for mm in mats])
        ms = t.time(5) / len(mats)
        byts = pbytes + m * k * 2 + m * n * 2
        sweep[f"{n}x{k}_m{m}"] = {"us": ms * 1e3, "gbs": byts / ms / 1e6,
                                  "frac_hbm": byts / ms / 1e6 / HBM_PEAK_GBS,
                                  "tflops": 2.0 * m * n * k / ms / 1e9}
        del t
    del mats, base
    torch.cuda.empty_cache()
    rows["gemm_small_batch_g128_f16"] = sweep

    # prefill GEMM M=2048, N=28672, K=8192 (+ its offline weight encode)
    w = torch.from_numpy(synth.prefill_weight()).to(dev)
    wp = rz.PackedTensor(rz.RAZER_WEIGHT, 28672, 8192, (-2, 4), dev)
    t = GraphTimer(torch, lambda: rz.razer_quantize_weight(w, out=wp))
    ms_q = t.time(5)
    # second-pair offset search on the same weight (15 full encodes + fp64 error sums)
    sse = torch.empty(len(rz.SECOND_PAIR_OFFSETS), dtype=torch.float64, device=dev)
    wso = torch.empty(rz.razer_workspace_bytes(rz.RAZER_OP_OFFSET_SEARCH, 0, 28672, 8192),
                      dtype=torch.uint8, device=dev)
    t = GraphTimer(torch, lambda: rz.razer_weight_offset_sse(w, -2, out=sse, workspace=wso))
    ms_o = t.time(3)
    sse_h = sse.cpu()
    best = rz.SECOND_PAIR_OFFSETS[int(torch.argmin(sse_h))]
    off_row = {"workload": "W [28672,8192] fp32, second-pair offsets -7..7 with the first pair at -2",
               "ms": ms_o, "gelem_per_s_per_offset": 15 * 28672 * 8192 / ms_o / 1e6,
               "best_offset": best,
               "sse_best_over_default_4": float(sse_h[best + 7] / sse_h[4 + 7])}
    # Four Over Six baseline encoder on the same weight: its encode time and
    # the relative squared error of each encoder on this weight
    wf = rz.PackedTensor(rz.RAZER_WEIGHT, 28672, 8192, (-2, 4), dev, rz.RAZER_FLAG_FOUR_OVER_SIX)
    t = GraphTimer(torch, lambda: rz.razer_quantize_weight(w, out=wf))
    ms_f = t.time(5)
    err_w = {"nvfp4": rel_sse(torch, rz, w, rz.razer_quantize_weight(w, (-2, 4), remap=False)),
             "four_over_six": rel_sse(torch, rz, w, wf),
             "razer_pairs_-2_4": rel_sse(torch, rz, w, wp),
             f"razer_pairs_-2_{best}": rel_sse(torch, rz, w, rz.razer_quantize_weight(w, (-2, best)))}
    # RaZeR with rescaled large special values on the same weight: its encode
    # time with the pairs (+-5, +-8), and the relative squared error for every
    # second-pair offset (the offset search composed from encodes and decodes)
    wr = rz.PackedTensor(rz.RAZER_WEIGHT, 28672, 8192, (-2, 4), dev, rz.RAZER_FLAG_RESCALE_LARGE_SV)
    t = GraphTimer(torch, lambda: rz.razer_quantize_weight(w, out=wr))
    ms_r = t.time(3)
    resc_sse = {o: rel_sse(torch, rz, w, rz.razer_quantize_weight(w, (-2, o), rescale=True))
                for o in rz.SECOND_PAIR_OFFSETS}
    best_r = min(resc_sse, key=lambda o: (resc_sse[o], o))
    resc_row = {"workload": "RaZeR with rescaled large special values (a candidate with |v| > 6 maps the block "
                            "maximum to |v|) on W [28672,8192] fp32: encode time with pairs (+-5, +-8), relative "
                            "squared error per second-pair offset (first pair at -2)",
                "ms": ms_r, "gelem_per_s": 28672 * 8192 / ms_r / 1e6,
                "rel_sse_by_offset": {str(o): v for o, v in resc_sse.items()},
                "best_offset": best_r, "rel_sse_best": resc_sse[best_r],
                "share_of_blocks_on_pair_1_at_+4": float(((wr.scales >> 6) & 1).float().mean()),
                "fixed_scale_best_rel_sse": err_w[f"razer_pairs_-2_{best}"]}
    del wr, t
    # layout variants (block sizes 16..128 with byte scales, and the FP16
    # group scale): relative squared error of each encoder on this weight, and
    # the RaZeR encode time of each layout
    var_w = {}
    for block, sfmt in ((16, 0), (32, 0), (64, 0), (128, 0), (128, 1), (16, 1)):
        name = f"b{block}_{'f16' if sfmt else 'byte'}"
        pv = rz.PackedTensor(rz.RAZER_WEIGHT, 28672, 8192, (-2, 4), dev, 0, block, sfmt)
        t = GraphTimer(torch, lambda: rz.razer_quantize_weight(w, out=pv))
        ms_v = t.time(3)
        var_w[name] = {
            "encode_ms": ms_v,
            "rel_sse": {
                "nvfp4": rel_sse(torch, rz, w, rz.razer_quantize_weight(w, (-2, 4), remap=False, block=block,
                                                                      scale_fmt=sfmt)),
                "four_over_six": rel_sse(torch, rz, w, rz.razer_quantize_weight(
                    w, (-2, 4), four_over_six=True, block=block, scale_fmt=sfmt)),
                "razer_pairs_-2_4": rel_sse(torch, rz, w, pv)}}
        del t, pv
    wg = rz.razer_quantize_weight(w, (-2, 4), block=128, scale_fmt=rz.RAZER_SCALE_F16)  # prefill, pages' layout
    del w, wso, wf
    torch.cuda.empty_cache()
    xa = synth.act_quant_x().to(dev)
    var_a = {}
    for block in (16, 32, 64, 128):
        var_a[f"b{block}_byte"] = {"rel_sse": {
            "nvfp4": rel_sse(torch, rz, xa, rz.razer_quantize_act(xa, remap=False, block=block)),
            "four_over_six": rel_sse(torch, rz, xa, rz.razer_quantize_act(xa, four_over_six=True, block=block)),
            "razer_pair_-2": rel_sse(torch, rz, xa, rz.razer_quantize_act(xa, block=block))}}
    err_a = {"nvfp4": rel_sse(torch, rz, xa, rz.razer_quantize_act(xa, remap=False)),
             "four_over_six": rel_sse(torch, rz, xa, rz.razer_quantize_act(xa, four_over_six=True)),
             "razer_pair_-2": rel_sse(torch, rz, xa, rz.razer_quantize_act(xa))}
    del xa
    torch.cuda.empty_cache()
    fos_row = {"workload": "Four Over Six encode of W [28672,8192] fp32; relative squared error "
                           "sum (x - dequant)^2 / sum x^2 of each encoder on that weight and on "
                           "X [4096,8192] bf16",
               "ms": ms_f, "gelem_per_s": 28672 * 8192 / ms_f / 1e6,
               "rel_sse_weight": err_w, "rel_sse_act": err_a}
    var_row = {"workload": "layout variants: RaZeR encode time of W [28672,8192] fp32 and the relative "
                           "squared error of NVFP4 / Four Over Six / RaZeR per layout on that weight and "
                           "on X [4096,8192] bf16 (the b16_byte encode time is the default kernel)",
               "weight": var_w, "act": var_a}
    x = synth.prefill_x().to(dev)
    y = torch.empty((2048, 28672), dtype=torch.bfloat16, device=dev)
    t = GraphTimer(torch, lambda: rz.razer_gemm(x, wp, out=y))
    ms = t.time(10)
    flops = 2.0 * 2048 * 28672 * 8192
    rows["gemm_prefill"] = {
        "workload": "x [2048,8192] bf16 x W [28672,8192] RaZeR-W4 (0.015*t(4)) -> bf16",
        "ms": ms, "tflops": flops / ms / 1e9, "frac_mfma": flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS}
    t = GraphTimer(torch, lambda: rz.razer_gemm(x, wg, out=y))
    ms = t.time(10)
    rows["gemm_prefill_g128_f16"] = {
        "workload": "the prefill product with W in 128-element blocks and FP16 scales",
        "ms": ms, "tflops": flops / ms / 1e9, "frac_mfma": flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS}
    del wg, t
    n_el = 28672 * 8192
    rows["offset_search_prefill"] = off_row
    rows["four_over_six_prefill"] = fos_row
    rows["rescale_large_sv_prefill"] = resc_row
    rows["layout_variants"] = var_row
    rows["quantize_weight_prefill"] = {
        "workload": "W [28672,8192] fp32, 4 candidates", "ms": ms_q, "gelem_per_s": n_el / ms_q / 1e6,
        "gbs_1read": n_el * (4 + 0.5625) / ms_q / 1e6,
        "frac_hbm_1read": n_el * (4 + 0.5625) / ms_q / 1e6 / HBM_PEAK_GBS}
    # W4A4 at the prefill shape: x encoded online (timed separately above), then
    # the product of the two packed tensors
    xq = rz.razer_quantize_act(x)
    w4 = torch.empty(rz.razer_workspace_bytes(rz.RAZER_OP_GEMM_W4A4, 2048, 28672, 8192), dtype=torch.uint8,
                     device=dev)
    t = GraphTimer(torch, lambda: rz.razer_gemm_w4a4(xq, wp, out=y, workspace=w4))
    ms_44 = t.time(10)
    rows["gemm_w4a4_prefill"] = {
        "workload": "RaZeR-A4 x [2048,8192] (from bf16 N(0,1)) x RaZeR-W4 W [28672,8192] -> bf16",
        "ms": ms_44, "tflops": flops / ms_44 / 1e9, "frac_mfma": flops / ms_44 / 1e9 / MFMA_BF16_PEAK_TFLOPS}
    del t, xq, w4
    out = torch.empty((28672, 8192), dtype=torch.bfloat16, device=dev)
    t = GraphTimer(torch, lambda: rz.razer_dequant(wp, out=out))
    ms_d = t.time(10)
    byts = packed_bytes(28672, 8192) + n_el * 2
    rows["dequant"] = {"workload": "W [28672,8192] -> bf16", "ms": ms_d, "gbs": byts / ms_d / 1e6,
                       "frac_hbm": byts / ms_d / 1e6 / HBM_PEAK_GBS}
    # Context for the prefill GEMM's MFMA fraction: the library's dense bf16
    # GEMM (torch.mm) on the same shape and the same (dequantized) weight
    # values, which decodes nothing.  The part is power-limited, so its rate
    # depends on the operands; this is the practical ceiling at these values.
    for _ in range(3):
        torch.mm(x, out.t(), out=y)
    torch.cuda.synchronize()
    settle(torch, lambda: torch.mm(x, out.t(), out=y))
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(10):
        torch.mm(x, out.t(), out=y)
    e1.record(st)
    e1.synchronize()
    ms_dense = e0.elapsed_time(e1) / 10
    rows["dense_bf16_gemm_ceiling"] = {
        "workload": "torch.mm bf16 x [2048,8192] x W^T, W [28672,8192] row-major (the dequantized RaZeR "
                    "weight of gemm_prefill) -> bf16; library GEMM, no decode",
        "ms": ms_dense, "tflops": flops / ms_dense / 1e9,
        "frac_mfma": flops / ms_dense / 1e9 / MFMA_BF16_PEAK_TFLOPS,
        "gemm_prefill_over_dense": rows["gemm_prefill"]["tflops"] / (flops / ms_dense / 1e9)}
    del t, x, y, wp, out
    torch.cuda.empty_cache()
    return rows


# ---- CPU oracle baseline ------------------------------------------------------------

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, layers):
    """The oracle's product over one decode step: `layers` passes over the
    layer's four GEMVs (the step's layer copies hold the same weights), on
    one host core: the calling thread is pinned to a single CPU while it runs."""
    import oracle

    names = ["qkv", "gate", "up", "down"]
    packs = {}
    for n in names:
        packs[n] = oracle.quantize_weight(synth.llama3_8b_decode_weight(n), (-2, 4))
    xs = {4096: synth.llama3_8b_decode_x(4096).float().numpy(),
          14336: synth.llama3_8b_decode_x(14336).float().numpy()}
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[-1]
    os.sched_setaffinity(0, {core})
    try:
        byts = 0
        t0 = time.perf_counter()
        for _ in range(layers):
            for n in names:
                p = packs[n]
                oracle.gemm(xs[p.cols], p)
                byts += gemv_bytes(p.rows, p.cols)
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, set(allowed))
    return {"value": byts / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"one decode step: {layers} x (qkv, gate, up, down GEMVs, 201M weights) of the "
                      "decode workload, weights encoded by the oracle (encode not timed), fp64 "
                      f"accumulation, {dt:.1f} s on one pinned core",
            "seconds": dt, "cpu_model": cpu_model(), "pinned_cpu": core,
            "host_cpus_visible": len(allowed)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--no-rows", action="store_true")
    ap.add_argument("--per-matrix", action="store_true",
                    help="one razer_gemv launch per matrix (gate and up not grouped)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--traffic-summary", nargs=6, metavar="CSV",
                    help="decode read, write, FETCH_SIZE CSVs, then the copy's three")
    ap.add_argument("--counters", choices=sorted(COUNTER_WORKLOADS),
                    help="run one workload's launches three times, untimed (for counter passes)")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import nvfp4_razer_w4a16_amd as rz
    from nvfp4_razer_w4a16_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    rz.lib()
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.copy_calibration:
        copy_calibration()
        return
    if args.counters:
        run_counter_workload(torch, rz, synth, args.counters)
        return

    log("decode: generating and encoding weights ...")
    steps, base = setup_decode(torch, rz, synth, args.layers)
    launches, step_bytes = steps["per_matrix" if args.per_matrix else "grouped"]
    if args.eager:  # counter passes: plain launches, nothing timed
        for _ in range(args.warmup + args.steps):
            run_launches(rz, launches)
        torch.cuda.synchronize()
        log(f"decode: {args.warmup + args.steps} eager steps of {len(launches)} launches")
        return
    timer = GraphTimer(torch, lambda: run_launches(rz, launches), warmup=1)
    for _ in range(args.warmup):
        timer.g.replay()
    torch.cuda.synchronize()
    settle_steps = settle(torch, timer.g.replay)  # untimed: the clocks settle
    ms_step = timer.time(args.steps, warmup=0, settle_ms=0)
    value = step_bytes / ms_step / 1e6  # GB/s
    log(f"decode: {ms_step * 1e3:.1f} us/step, {value:.0f} GB/s")

    # live per-kernel figure for the GEMV kernel: the same launches, timed as one
    # graph on the launch stream; average duration per launch = elapsed / launches
    n_launch = len(launches)
    avg_us = ms_step * 1e3 / n_launch
    bytes_per_launch = step_bytes / n_launch
    achieved = bytes_per_launch / (avg_us * 1e-6) / 1e9
    src = source_hash(*DECODE_SOURCES)
    traffic = load_traffic("gemv_decode", src)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": ("razer_gemv: gemv_kernel (qkv, gate, up) + smallm_kernel (down)" if args.per_matrix
                           else "razer_gemv (qkv: gemv_kernel; down: smallm_kernel) + razer_gemv_group "
                                "(gate and up: one gemv_kernel launch)"),
                "avg_launch_us": round(avg_us, 3),
                "algorithmic_bytes_per_launch": bytes_per_launch}

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if not args.per_matrix:
        roofline["per_kernel"] = per_kernel_rates(torch, rz, launches, args.steps)
    floor = step_read_floor(torch, launches, step_bytes, args.steps)
    roofline["step_read_floor_us"] = round(floor["us_per_step"], 2)
    roofline["frac_of_step_read_floor"] = round(floor["us_per_step"] / (ms_step * 1e3), 4)
    log(f"decode: read floor {floor['us_per_step']:.1f} us/step; per kernel "
        + ", ".join(f"{k} {v['avg_launch_us']:.2f} us ({v['frac']:.2f})" for k, v in roofline.get("per_kernel", {}).items()))

    rows = None
    if not args.no_rows:
        # the other launch arrangement of the same step, for comparison
        other = "grouped" if args.per_matrix else "per_matrix"
        l2, b2 = steps[other]
        ms2 = GraphTimer(torch, lambda: run_launches(rz, l2), warmup=1).time(args.steps)
        decode_other = {"workload": f"the same decode step, {other.replace('_', ' ')} launches",
                        "launches_per_step": len(l2), "us_per_step": ms2 * 1e3, "gbs": b2 / ms2 / 1e6,
                        "frac_hbm": b2 / ms2 / 1e6 / HBM_PEAK_GBS}
        # the same step with the weights in the pages' kernel layout (128-element
        # blocks, FP16 scales with the metadata in the sign and top exponent bits)
        del l2
        steps_g, _ = setup_decode(torch, rz, synth, args.layers, block=128, scale_fmt=rz.RAZER_SCALE_F16)
        l3, b3 = steps_g["grouped"]
        ms3 = GraphTimer(torch, lambda: run_launches(rz, l3), warmup=1).time(args.steps)
        decode_g128 = {"workload": "the same decode step (grouped launches) with 128-element blocks and FP16 "
                                   "scales (0.5156 B per weight)", "launches_per_step": len(l3),
                       "us_per_step": ms3 * 1e3, "gbs": b3 / ms3 / 1e6, "frac_hbm": b3 / ms3 / 1e6 / HBM_PEAK_GBS,
                       "bytes_per_step": b3}
        del steps_g, l3
        torch.cuda.empty_cache()
        log("rows: encoders, small-batch sweep, prefill ...")
        # the same grouped step with the untrimmed launch plan (every CU, the most
        # K splits, one row quad per wave): what the per-shape launch sizing gains
        lu = [(x, [w.with_flags(rz.RAZER_FLAG_UNTRIMMED_PLAN) for w in ws], ys) for x, ws, ys in launches]
        ms_u = GraphTimer(torch, lambda: run_launches(rz, lu), warmup=1).time(args.steps)
        decode_untrimmed = {"workload": "the same decode step with the untrimmed launch plan",
                            "us_per_step": ms_u * 1e3, "gbs": step_bytes / ms_u / 1e6,
                            "plan_gain_pct": 100.0 * (ms_u - ms_step) / ms_u}
        del lu
        rows = {f"decode_{other}": decode_other, "decode_g128_f16": decode_g128,
                "decode_untrimmed_plan": decode_untrimmed,
                "decode_step_read_floor": floor, "mfma_loop_ceiling": mfma_loop_ceiling(torch, cus)}
        rows.update(bench_rows(torch, rz, synth, args, base))
        pf, ml = rows["gemm_prefill"], rows["mfma_loop_ceiling"]
        pf["frac_of_mfma_loop"] = pf["tflops"] / ml["tflops"]

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on one decode step ...")
        cpu = cpu_baseline(synth, args.layers)
        cpu["value"] = round(cpu["value"], 4)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "settle": {"ms": SETTLE_MS, "untimed_steps": settle_steps},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic (seeded Philox; Student-t(5)*0.02 weights, N(0,1) fp16 x with 8 channels x20)",
        "config": {"workload": f"llama3-8b decode GEMV: qkv 6144x4096, gate 14336x4096, "
                               f"up 14336x4096, down 4096x14336; M=1; {args.layers} layer copies; "
                               "RaZeR-W4 weights, fp16 x and y"
                               + ("" if args.per_matrix else "; gate and up (same x) in one launch"),
                   "layers": args.layers, "m": 1, "launches_per_step": n_launch,
                   "bytes_per_step": step_bytes},
        "roofline": roofline, "cpu_baseline": cpu, "rows": rows,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
