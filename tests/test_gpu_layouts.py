"""razer_gemm on the pages' kernel layout -- 128-element blocks whose FP16
scale carries the metadata in its sign and top exponent bits -- for every
batch size: small batches, the generic tile kernel and the prefill kernel,
against the oracle's fp64 product over its own decoded weights (gemm_any),
within 2e-3 * sum |x||w| per output."""
import functools

import numpy as np
import pytest
import torch

import nvfp4_razer_w4a16_amd as rz
import oracle
from nvfp4_razer_w4a16_amd import synth

from gpu_common import _need_gpu, as_f32, assert_product_close, log, to_device

pytestmark = pytest.mark.gpu


def _f16s_weight(n, k, seed, offsets=(-2, -5)):
    rng = np.random.default_rng(seed)
    w = (rng.standard_t(5, (n, k)) * 0.02).astype(np.float32)
    return oracle.quantize(oracle.WEIGHT, w, offsets, block=128, scale_fmt=oracle.SCALE_F16)


@pytest.mark.parametrize("m,n,k,xdt", [(2, 300, 1024, torch.bfloat16), (3, 96, 640, torch.float16),
                                       (8, 520, 2048, torch.bfloat16), (16, 64, 4096, torch.float16),
                                       (17, 130, 384, torch.bfloat16), (32, 4100, 1024, torch.bfloat16),
                                       (100, 257, 512, torch.float16), (300, 260, 1152, torch.bfloat16),
                                       (256, 96, 128, torch.float16), (4, 1000, 4096, torch.float16),
                                       (5, 77, 768, torch.bfloat16), (6, 200, 256, torch.float16),
                                       (7, 33, 1280, torch.bfloat16), (10, 8320, 1024, torch.float16),
                                       (16, 8200, 512, torch.bfloat16), (24, 16400, 512, torch.float16),
                                       (9, 200, 768, torch.bfloat16)])
def test_gemm_group128_f16_layout(m, n, k, xdt):
    _need_gpu()
    ref = _f16s_weight(n, k, m * 131 + n + k)
    rng = np.random.default_rng(m + n * k)
    x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(xdt)
    y_ref, nrm = oracle.gemm_any(as_f32(x), ref)
    t = to_device(ref)
    for odt in (torch.float32, torch.bfloat16):
        y = rz.razer_gemm(x.cuda(), t, odt).float().cpu().numpy()
        assert_product_close(y, y_ref, nrm, f"g128 gemm {m}x{n}x{k} out {odt}", odt)


@functools.lru_cache(maxsize=1)
def _prefill_f16s():
    log("g128 prefill: generating W ...")
    w = synth.prefill_weight()
    log("g128 prefill: oracle encode ...")
    return oracle.quantize(oracle.WEIGHT, w, (-2, 4), block=128, scale_fmt=oracle.SCALE_F16)


@pytest.mark.parametrize("m", [3, 8, 12, 32, 2048])
def test_gemm_group128_f16_layout_full_size_sampled(m):
    """The prefill weight W[28672, 8192] in the 128-element FP16 layout, with
    8 rows (small batch) and 2048 rows (prefill), on 257 columns that cover
    every position inside a 256-wide output tile, bf16 output."""
    _need_gpu()
    ref = _prefill_f16s()
    t = to_device(ref)
    x = synth.prefill_x()[:m]
    rng = np.random.default_rng(128 + m)
    cols = np.unique(np.append(np.arange(256) + 256 * rng.integers(0, 112, 256), 28671))
    log(f"g128 m={m}: oracle on {cols.size} columns ...")
    y_ref, nrm = oracle.gemm_any(as_f32(x), ref, cols)
    y = rz.razer_gemm(x.cuda(), t, torch.bfloat16)
    torch.cuda.synchronize()
    yc = y[:, torch.from_numpy(cols).cuda()].float().cpu().numpy()
    e = assert_product_close(yc, y_ref, nrm, f"g128 gemm m={m} 28672x8192", torch.bfloat16)
    assert torch.isfinite(y).all()
    log(f"g128 m={m}: max err/norm {e:.2e}")


# ---- untrimmed launch plan (RAZER_FLAG_UNTRIMMED_PLAN) ------------------------------

@pytest.mark.parametrize("m,n,k", [(1, 6144, 4096), (1, 28672, 4096), (1, 4096, 14336), (2, 4096, 4096),
                                   (4, 4096, 4096), (8, 4096, 4096), (32, 4096, 4096), (16, 600, 8192)])
def test_untrimmed_plan_matches_the_oracle(m, n, k):
    """The products launched with the untrimmed plan (every CU, the most K
    splits) stay within tolerance of the oracle; only the summation order
    differs from the tuned plan."""
    _need_gpu()
    rng = np.random.default_rng(n + k + m)
    w = (rng.standard_t(5, (n, k)) * 0.02).astype(np.float32)
    ref = oracle.quantize_weight(w, (-2, -5))
    x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    cols = np.unique(np.append(rng.choice(n, min(n, 300), replace=False), n - 1))
    y_ref, nrm = oracle.gemm(as_f32(x), ref, cols)
    t = to_device(ref).with_flags(rz.RAZER_FLAG_UNTRIMMED_PLAN)
    y = rz.razer_gemm(x.cuda(), t, torch.float32)
    torch.cuda.synchronize()
    yc = y[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    assert_product_close(yc, y_ref, nrm, f"untrimmed {m}x{n}x{k}")
    if m == 1:
        yg = rz.razer_gemv(x.cuda().reshape(-1), t, torch.float32)
        assert torch.equal(yg, y[0])


@pytest.mark.parametrize("m,n,k", [(4, 2048, 1024), (12, 2100, 768), (6, 300, 4096)])
def test_untrimmed_plan_on_the_fp16_scale_layout(m, n, k):
    """The FP16-scale products with the untrimmed plan (one tile and eight K
    slices per workgroup on the streaming kernel) stay within tolerance of the
    oracle, and so does the tuned plan on the same operands."""
    _need_gpu()
    ref = _f16s_weight(n, k, 7 * m + n + k, offsets=(-2, 4))
    rng = np.random.default_rng(m + 3 * n + k)
    x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    y_ref, nrm = oracle.gemm_any(as_f32(x), ref)
    t = to_device(ref)
    for tt in (t, t.with_flags(rz.RAZER_FLAG_UNTRIMMED_PLAN)):
        y = rz.razer_gemm(x.cuda(), tt, torch.float32).cpu().numpy()
        assert_product_close(y, y_ref, nrm, f"g128 untrimmed {m}x{n}x{k}")


def test_encoders_reject_the_untrimmed_flag():
    _need_gpu()
    x = torch.randn(16, 64, device="cuda")
    out = rz.PackedTensor(rz.RAZER_WEIGHT, 16, 64, (-2, 4), "cuda", rz.RAZER_FLAG_UNTRIMMED_PLAN)
    with pytest.raises(rz.RazerError) as e:
        rz.razer_quantize_weight(x, out=out)
    assert e.value.status == rz.RAZER_E_INVALID
