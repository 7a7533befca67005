"""GPU parity at the full sizes the bench times, and in the launch
configurations the bench uses.

- razer_gemm with one and sixteen activation rows on W[28672, 8192] (the
  vector GEMV with a four-way K split, and the batch kernel), f32 and bf16
  outputs, on sampled columns;
- the vector GEMV on rows above 4096 with K = 4128 .. 16416, which covers its
  four-way K split with one, two and four chunks per lane;
- every full-size weight (the decode layer's four and the prefill weight)
  encoded with a second pair that is actually selected (offsets (-2, -5),
  special values +-5 and +-3.5), bit for bit;
- the prefill and W4A4 prefill products on 256 columns, one at every position
  inside the 256-wide output tile, for bf16 and f32 outputs, plus 4096 random
  (m, n) outputs of the whole product.

Expected values come from the oracle only (its own encodings of the seeded
inputs, its fp64 products).
"""
import functools

import numpy as np
import pytest
import torch

import nvfp4_razer_w4a16_amd as rz
import oracle
from nvfp4_razer_w4a16_amd import synth

from gpu_common import (_need_gpu, as_f32, assert_product_close, assert_same_encoding, gpu_encode,
                        llama_weight, log, prefill_weight_packed, small_batch_ref, to_device)

pytestmark = pytest.mark.gpu

N70, K70 = 28672, 8192


def tile_columns(n, seed, tile=256):
    """One column at every position inside a `tile`-wide output tile, each in a
    random tile, plus the last column."""
    rng = np.random.default_rng(seed)
    ntile = n // tile
    cols = np.arange(tile) + tile * rng.integers(0, ntile, tile)
    return np.unique(np.append(cols, n - 1))


@functools.lru_cache(maxsize=1)
def _w70_device():
    return to_device(small_batch_ref(N70, K70))


@pytest.mark.parametrize("m", [1, 16])
def test_gemm_70b_one_and_sixteen_rows_sampled(m):
    """M = 1 runs the vector GEMV (two 32-element chunks per lane pair, K split
    four ways), M = 16 the batch kernel; both against the oracle on 257
    columns, with f32 and bf16 outputs."""
    _need_gpu()
    log(f"gemm 70b m={m}: reference encode ...")
    ref = small_batch_ref(N70, K70)
    t = _w70_device()
    x = synth.small_batch_x(m, K70)
    cols = tile_columns(N70, 700 + m)
    log(f"gemm 70b m={m}: oracle on {cols.size} columns ...")
    y_ref, nrm = oracle.gemm(as_f32(x), ref, cols)
    for odt in (torch.float32, torch.bfloat16):
        y = rz.razer_gemm(x.cuda(), t, odt)
        torch.cuda.synchronize()
        yc = y[:, torch.from_numpy(cols).cuda()].float().cpu().double().numpy()
        e = assert_product_close(yc, y_ref, nrm, f"gemm m={m} 28672x8192 out {odt}", odt)
        assert torch.isfinite(y).all()
        log(f"gemm 70b m={m} out {odt}: max err/norm {e:.2e}")


@pytest.mark.parametrize("n,k,xdt", [(4100, 4128, torch.float16), (4352, 8192, torch.bfloat16),
                                     (5000, 12320, torch.float16), (4097, 16416, torch.bfloat16)])
def test_gemv_long_rows_four_way_k_split(n, k, xdt):
    """More than 4096 rows keeps these on the vector GEMV; K = 4128 .. 16416
    makes it split K over four waves with one (4128, 8192), two (12320) or
    four (16416) chunks per lane, with ragged tails of K and of the rows."""
    _need_gpu()
    rng = np.random.default_rng(n + 3 * k)
    w = (rng.standard_t(5, (n, k)) * 0.02).astype(np.float32)
    x = torch.from_numpy(rng.normal(0, 1, k).astype(np.float32)).to(xdt)
    ref = oracle.quantize_weight(w, (-2, -5))
    y_ref, nrm = oracle.gemm(as_f32(x)[None, :], ref)
    t = to_device(ref)
    for odt in (torch.float32, torch.float16):
        y = rz.razer_gemv(x.cuda(), t, odt).float().cpu().double().numpy()
        e = assert_product_close(y[None, :], y_ref, nrm, f"gemv {n}x{k} out {odt}", odt)
        log(f"gemv {n}x{k} {xdt} out {odt}: max err/norm {e:.2e}")


@pytest.mark.parametrize("name", ["qkv", "gate", "up", "down"])
def test_decode_weights_with_selected_second_pair(name):
    """The decode layer's weights at full size with the second pair at +-3.5
    (offset -5), which a large share of the blocks selects."""
    _need_gpu()
    w = llama_weight(name)
    log(f"{name} (-2,-5): oracle encode ...")
    ref = oracle.quantize_weight(w, (-2, -5))
    p = gpu_encode(oracle.WEIGHT, torch.from_numpy(w), (-2, -5))
    assert_same_encoding(p, ref, None, f"llama {name} weight (-2, -5)")
    pair = (ref.scales >> 6) & 1
    log(f"{name} (-2,-5): blocks on the second pair {pair.mean():.3f}")
    assert pair.any()


def test_prefill_weight_with_selected_second_pair():
    _need_gpu()
    log("prefill W (-2,-5): generating ...")
    w = synth.prefill_weight()
    log("prefill W (-2,-5): oracle encode ...")
    ref = oracle.quantize_weight(w, (-2, -5))
    log("prefill W (-2,-5): gpu ...")
    p = gpu_encode(oracle.WEIGHT, torch.from_numpy(w), (-2, -5))
    assert_same_encoding(p, ref, None, "prefill weight (-2, -5)")
    sel = (ref.scales >> 6) & 3
    log(f"prefill W (-2,-5): selections {np.bincount(sel, minlength=4).tolist()}")
    assert (sel >= 2).any()
    del p
    torch.cuda.empty_cache()


def _random_pairs(m, n, count, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, m, count), rng.integers(0, n, count)


def test_gemm_prefill_every_tile_column_and_random_outputs():
    """Prefill M=2048, N=28672, K=8192: 257 columns (every position inside the
    256-wide output tile) x all 2048 rows (every position inside the 256-row
    tile), for bf16 and f32 outputs, and 4096 random outputs of the f32 run."""
    _need_gpu()
    ref = prefill_weight_packed()
    t = to_device(ref)
    x = synth.prefill_x()
    xd = x.cuda()
    cols = tile_columns(N70, 2048)
    log(f"prefill: oracle on {cols.size} columns x 2048 rows ...")
    y_ref, nrm = oracle.gemm(as_f32(x), ref, cols)
    ci = torch.from_numpy(cols).cuda()
    for odt in (torch.bfloat16, torch.float32):
        log(f"prefill: gpu gemm out {odt} ...")
        y = rz.razer_gemm(xd, t, odt)
        torch.cuda.synchronize()
        yc = y[:, ci].float().cpu().double().numpy()
        e = assert_product_close(yc, y_ref, nrm, f"prefill out {odt} (tile columns)", odt)
        assert torch.isfinite(y).all()
        log(f"prefill out {odt}: max err/norm {e:.2e}")
    mi, ni = _random_pairs(2048, N70, 4096, 4096)
    log("prefill: oracle on 4096 random outputs ...")
    yp, np_ = oracle.gemm_pairs(as_f32(x), ref, mi, ni)
    got = y[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().double().numpy()
    assert_product_close(got, yp, np_, "prefill out f32 (random outputs)")


@pytest.mark.parametrize("m,n,k,xdt", [(505, 256 * 130 - 100, 128, torch.bfloat16),
                                       (300, 256 * 129 + 1, 192, torch.float16)])
def test_gemm_prefill_tail_split_ragged(m, n, k, xdt):
    """260 tiles of 256x256 on 256 compute units: the last four tiles run as two
    K halves (one and one, or one and two K steps) folded by a second launch.
    Those tiles hold the ragged last rows and columns.  Checked against the
    oracle on every column of the tail tiles plus sampled others, for f32 and
    bf16 outputs, with the workspace (split) and with a 16-byte one (unsplit)."""
    _need_gpu()
    rng = np.random.default_rng(m + n + k)
    w = (rng.standard_t(4, (n, k)) * 0.015).astype(np.float32)
    x = torch.from_numpy(rng.normal(0, 1, (m, k)).astype(np.float32)).to(xdt)
    ref = oracle.quantize_weight(w, (-2, -5))
    ntn = (n + 255) // 256
    tiles = ((m + 255) // 256) * ntn
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tail = tiles % cus if tiles > cus and 2 * (tiles % cus) <= cus else 0
    first = (tiles - tail) % ntn * 256 if tail else n
    cols = np.unique(np.concatenate([np.arange(first, n), rng.choice(first, 64, replace=False)]))
    need = rz.razer_workspace_bytes(rz.RAZER_OP_GEMM, m, n, k)
    log(f"tail split {m}x{n}x{k}: {tiles} tiles, {tail} split, workspace {need} bytes, "
        f"{cols.size} columns checked")
    assert need == tail * 2 * 256 * 256 * 4
    y_ref, nrm = oracle.gemm(as_f32(x), ref, cols)
    t = to_device(ref)
    ci = torch.from_numpy(cols).cuda()
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    for odt in (torch.float32, torch.bfloat16):
        for ws in (None, small):
            y = rz.razer_gemm(x.cuda(), t, odt, workspace=ws)
            torch.cuda.synchronize()
            got = y[:, ci].float().cpu().double().numpy()
            what = f"prefill tail {m}x{n}x{k} out {odt} " + ("split" if ws is None else "unsplit")
            assert_product_close(got, y_ref, nrm, what, odt)
            assert torch.isfinite(y).all(), what


def test_gemm_w4a4_prefill_every_tile_column_and_random_outputs():
    """W4A4 at the prefill shape: the activation encoded by the oracle, the
    same tile columns and random outputs as the W4A16 prefill, bf16 and f32."""
    _need_gpu()
    wp = prefill_weight_packed()
    log("w4a4 prefill: oracle act encode ...")
    xp = oracle.quantize_act(synth.prefill_x().float().numpy(), (-2,))
    xt, wt = to_device(xp), to_device(wp)
    cols = tile_columns(N70, 4404)
    log(f"w4a4 prefill: oracle on {cols.size} columns ...")
    y_ref, nrm = oracle.gemm_w4a4(xp, wp, cols)
    ci = torch.from_numpy(cols).cuda()
    for odt in (torch.bfloat16, torch.float32):
        log(f"w4a4 prefill: gpu out {odt} ...")
        y = rz.razer_gemm_w4a4(xt, wt, odt)
        torch.cuda.synchronize()
        yc = y[:, ci].float().cpu().double().numpy()
        e = assert_product_close(yc, y_ref, nrm, f"w4a4 prefill out {odt} (tile columns)", odt)
        assert torch.isfinite(y).all()
        log(f"w4a4 prefill out {odt}: max err/norm {e:.2e}")
    mi, ni = _random_pairs(2048, N70, 4096, 4405)
    yp, np_ = oracle.gemm_w4a4_pairs(xp, wp, mi, ni)
    got = y[torch.from_numpy(mi).cuda(), torch.from_numpy(ni).cuda()].cpu().double().numpy()
    assert_product_close(got, yp, np_, "w4a4 prefill out f32 (random outputs)")
