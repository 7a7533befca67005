"""GPU parity: librazer (HIP, through the C ABI) against the CPU oracle.

Encodings (codes, scale bytes, tensor scale) and dequantized values must match
bit for bit.  Products must satisfy |y - y_ref| <= 2e-3 * sum_k |x| |w| per
output, with y_ref the oracle's fp64 product over the oracle's own packed
weights.  Inputs come from the seeded generators in nvfp4_razer_w4a16_amd.synth;
no expected value comes from the GPU path.
"""
import functools

import numpy as np
import pytest
import torch

import nvfp4_razer_w4a16_amd as rz
import oracle
from nvfp4_razer_w4a16_amd import synth

from gpu_common import (OUT_MANT_BITS, TOL, _need_gpu, as_f32, assert_product_close,  # noqa: F401
                        assert_same_encoding, gpu_encode, llama_ref, llama_weight, log, pr1,
                        prefill_weight_packed as _prefill_weight_packed, small_batch_ref, to_device)

pytestmark = pytest.mark.gpu


# ---- encoder parity ------------------------------------------------------------

@pytest.mark.parametrize("offsets", [(-2, 4), (-2, -5), (-7, 7), (0, -1)])
def test_quantize_weight_pr1(offsets):
    _need_gpu()
    w, _ = pr1()
    ref = oracle.quantize_weight(w.numpy(), offsets)
    p = gpu_encode(oracle.WEIGHT, w, offsets)
    assert_same_encoding(p, ref, w.numpy(), f"pr1 offsets {offsets}")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_quantize_weight_16bit_inputs(dtype):
    _need_gpu()
    w, _ = pr1()
    w16 = w.to(dtype)
    ref = oracle.quantize_weight(as_f32(w16), (-2, -5))
    p = gpu_encode(oracle.WEIGHT, w16, (-2, -5))
    assert_same_encoding(p, ref, as_f32(w16), f"weights in {dtype}")


def test_quantize_no_remap_is_plain_nvfp4():
    _need_gpu()
    w, _ = pr1()
    ref = oracle.quantize_weight(w.numpy(), (-2, 4), remap=False)
    p = gpu_encode(oracle.WEIGHT, w, (-2, 4), remap=False)
    assert_same_encoding(p, ref, w.numpy(), "no remap")
    assert not (p.scales.cpu() & 0xC0).any()


def _edge_tensors():
    rng = np.random.default_rng(101)
    cases = {}
    cases["one_block"] = rng.normal(0, 1, (1, 16)).astype(np.float32)
    cases["ragged_rows_cols"] = rng.normal(0, 0.02, (7, 48)).astype(np.float32)
    cases["zeros"] = np.zeros((4, 64), np.float32)
    t = rng.normal(0, 1, (8, 64)).astype(np.float32)
    t[3, 17] = np.nan
    cases["nan"] = t
    t = rng.normal(0, 1, (8, 64)).astype(np.float32)
    t[0, 0] = -np.inf
    cases["inf"] = t
    cases["tiny_subnormal"] = (rng.normal(0, 1, (4, 64)) * 1e-40).astype(np.float32)
    cases["huge"] = (rng.normal(0, 1, (4, 64)) * 1e37).astype(np.float32)
    t = rng.normal(0, 1, (16, 64)).astype(np.float32)
    t[2, :16] *= 1e-6      # block underflows to scale code 0
    t[5, 16:32] *= 1e-3    # subnormal scale codes
    t[9, 32:48] = 0.0      # all-zero block
    t[11, 0] = 1e4         # one dominant element
    cases["mixed_blocks"] = t
    # values placed on exact decision points after scaling (block max 6 * D)
    t = np.zeros((4, 64), np.float32)
    pts = np.array([6, 5, 4.5, 5.5, 4.75, 5.25, 2.25, 2.75, 3.25, 3.75, 0.25, 0.75, 1.25, 1.75,
                    2.5, 3.5], np.float32)
    for r in range(4):
        t[r] = np.tile(pts * (1 if r % 2 else -1), 4)
    cases["decision_points"] = t
    cases["all_equal"] = np.full((2, 32), 0.37, np.float32)
    return cases


EDGE = _edge_tensors()


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("kind,offsets", [(oracle.WEIGHT, (-2, -5)), (oracle.ACT, (-2,))])
def test_quantize_edge_cases(name, kind, offsets):
    _need_gpu()
    x = EDGE[name]
    ref = oracle.quantize(kind, x, offsets)
    p = gpu_encode(kind, torch.from_numpy(x), offsets)
    assert_same_encoding(p, ref, x, f"edge {name} kind {kind}")


def test_quantize_empty_tensor():
    _need_gpu()
    x = torch.zeros((0, 32), device="cuda")
    p = rz.razer_quantize_weight(x)
    torch.cuda.synchronize()
    assert float(p.tensor_scale.cpu()[0]) == 0.0


def test_quantize_weight_every_second_pair_offset():
    _need_gpu()
    rng = np.random.default_rng(55)
    w = rng.standard_t(5, (32, 256)).astype(np.float32) * 0.02
    wt = torch.from_numpy(w)
    for off in range(-7, 8):
        ref = oracle.quantize_weight(w, (-2, off))
        p = gpu_encode(oracle.WEIGHT, wt, (-2, off))
        assert_same_encoding(p, ref, w, f"second pair offset {off}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_quantize_act_parity(dtype):
    _need_gpu()
    x = synth.act_quant_x(256, 8192).to(dtype)
    ref = oracle.quantize_act(as_f32(x))
    p = gpu_encode(oracle.ACT, x, (-2,))
    assert_same_encoding(p, ref, as_f32(x), f"act {dtype}")


def _e4m3_boundary_blocks(dtype, tensor_max, seed):
    """Blocks whose maximum sits on every E4M3 rounding midpoint of
    448 * amax_b / amax, and one step of the input type either side."""
    vals = np.array([c * 2.0 ** -9 if c < 8 else (8 + (c & 7)) * 2.0 ** ((c >> 3) - 10)
                     for c in range(127)])
    mids = (vals[:-1] + vals[1:]) / 2
    base = torch.from_numpy((mids * tensor_max / 448.0).astype(np.float32)).to(dtype)
    bits = base.view(torch.int16)
    tops = torch.cat([bits - 1, bits, bits + 1]).view(dtype).float().numpy()
    rng = np.random.default_rng(seed)
    blocks = rng.uniform(-0.5, 0.5, (tops.size + 1, 16)) * np.append(tops, tensor_max)[:, None]
    blocks[:-1, 0] = tops * np.where(rng.integers(0, 2, tops.size) == 1, -1.0, 1.0)
    blocks[-1, 3] = tensor_max
    rows = -(-blocks.size // 64)
    x = np.zeros(rows * 64, np.float32)
    x[:blocks.size] = blocks.reshape(-1)
    return torch.from_numpy(x.reshape(rows, 64)).to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("tensor_max", [448.0, 1.0, 37.25])
def test_quantize_act_scale_code_boundaries(dtype, tensor_max):
    """Block maxima on every E4M3 rounding midpoint (and one input step either
    side) give the oracle's scale byte: the activation encoder forms the block
    ratio with a corrected reciprocal product and rounds it with the fp8
    conversion for 16-bit inputs."""
    _need_gpu()
    x = _e4m3_boundary_blocks(dtype, tensor_max, seed=int(tensor_max * 8))
    ref = oracle.quantize_act(as_f32(x))
    p = gpu_encode(oracle.ACT, x, (-2,))
    assert_same_encoding(p, ref, as_f32(x), f"act scale boundaries {dtype} max {tensor_max}")


def test_quantize_act_full_size():
    """Activation quantizer at its full size, X[4096, 8192] bf16."""
    _need_gpu()
    x = synth.act_quant_x()
    log("act full: oracle ...")
    ref = oracle.quantize_act(as_f32(x))
    log("act full: gpu ...")
    p = gpu_encode(oracle.ACT, x, (-2,))
    assert_same_encoding(p, ref, None, "act full size")
    sel = (p.scales.cpu().numpy() >> 7)
    log(f"act full: blocks selecting -5: {sel.mean():.3f}")


def test_quantize_weight_prefill_full_size():
    """Weight quantizer at its full size, W[28672, 8192] fp32 ~ 0.015 t(4)."""
    _need_gpu()
    log("prefill W: generating ...")
    w = synth.prefill_weight()
    log("prefill W: oracle ...")
    ref = oracle.quantize_weight(w)
    log("prefill W: gpu ...")
    p = gpu_encode(oracle.WEIGHT, torch.from_numpy(w), (-2, 4))
    assert_same_encoding(p, ref, None, "prefill weight full size")
    del p
    torch.cuda.empty_cache()


def test_quantize_deterministic_across_calls():
    _need_gpu()
    w, _ = pr1()
    a = gpu_encode(oracle.WEIGHT, w, (-2, -5))
    b = gpu_encode(oracle.WEIGHT, w, (-2, -5))
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)


# ---- Four Over Six baseline encoder ----------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("kind", [oracle.WEIGHT, oracle.ACT])
def test_quantize_four_over_six_parity(kind, dtype):
    _need_gpu()
    if kind == oracle.WEIGHT:
        x, offs = pr1()[0].to(dtype), (-2, 4)
    else:
        x, offs = synth.act_quant_x(128, 4096).to(dtype), (-2,)
    ref = oracle.quantize(kind, as_f32(x), offs, four_over_six=True)
    p = gpu_encode(kind, x, offs, four_over_six=True)
    assert_same_encoding(p, ref, as_f32(x), f"four over six kind {kind} {dtype}")
    s = p.scales.cpu().numpy()
    assert not (s >> (6 if kind == oracle.WEIGHT else 7)).any()  # no metadata bits
    c = p.codes.cpu().numpy()
    assert not ((c & 15) == 8).any() and not ((c >> 4) == 8).any()  # never the special code


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("kind,offsets", [(oracle.WEIGHT, (-2, -5)), (oracle.ACT, (-2,))])
def test_quantize_four_over_six_edge_cases(name, kind, offsets):
    _need_gpu()
    x = EDGE[name]
    ref = oracle.quantize(kind, x, offsets, four_over_six=True)
    p = gpu_encode(kind, torch.from_numpy(x), offsets, four_over_six=True)
    assert_same_encoding(p, ref, x, f"four over six edge {name} kind {kind}")


def test_quantize_four_over_six_takes_precedence_over_no_remap():
    _need_gpu()
    w = pr1()[0]
    ref = oracle.quantize_weight(w.numpy(), (-2, 4), four_over_six=True)
    out = rz.PackedTensor(rz.RAZER_WEIGHT, w.shape[0], w.shape[1], (-2, 4), "cuda",
                          rz.RAZER_FLAG_FOUR_OVER_SIX | rz.RAZER_FLAG_NO_REMAP)
    rz.razer_quantize_weight(w.cuda(), (-2, 4), out=out)
    torch.cuda.synchronize()
    assert_same_encoding(out, ref, w.numpy(), "four over six | no remap")


def test_quantize_four_over_six_prefill_weight_sampled():
    """Four Over Six on the full W[28672, 8192] fp32 weight: every block's
    encoding depends only on the block and the tensor scale, so the oracle
    encodes a row sample together with the row holding the tensor maximum
    (same tensor scale) and the GPU rows must match it byte for byte."""
    _need_gpu()
    w = synth.prefill_weight()
    log("4/6 prefill W: gpu ...")
    p = gpu_encode(oracle.WEIGHT, torch.from_numpy(w), (-2, 4), four_over_six=True)
    rmax = int(np.abs(w).max(axis=1).argmax())
    rows = sorted(set(np.random.default_rng(91).choice(w.shape[0], 96, replace=False).tolist()) | {rmax, 0, w.shape[0] - 1})
    log("4/6 prefill W: oracle on", len(rows), "rows ...")
    ref = oracle.quantize_weight(w[rows], (-2, 4), four_over_six=True)
    k = w.shape[1]
    codes = p.codes.cpu().numpy().reshape(w.shape[0], k // 2)[rows]
    scales = p.scales.cpu().numpy().reshape(w.shape[0], k // 16)[rows]
    ts = p.tensor_scale.cpu().numpy().view(np.uint32)[0]
    assert ts == np.array([ref.tensor_scale], np.float32).view(np.uint32)[0]
    np.testing.assert_array_equal(scales.reshape(-1), ref.scales)
    np.testing.assert_array_equal(codes.reshape(-1), ref.codes)
    frac4 = float(np.mean(scales != oracle.quantize_weight(w[rows], (-2, 4), remap=False).scales.reshape(scales.shape)))
    log(f"4/6 prefill W: blocks taking max -> 4: {frac4:.3f}")
    del p
    torch.cuda.empty_cache()


def _rescale_input(kind, dtype, seed):
    rng = np.random.default_rng(seed)
    if kind == oracle.WEIGHT:
        x = (rng.standard_t(5, (48, 512)) * 0.02).astype(np.float32)
    else:
        x = rng.standard_normal((48, 512)).astype(np.float32)
        x[:, 9] *= 30
    return torch.from_numpy(x).to(dtype)


# activations come in 16-bit types only
_RESCALE_CASES = [(kind, offsets, dtype)
                  for kind, offsets in [(oracle.WEIGHT, (-2, 4)), (oracle.WEIGHT, (-2, 2)),
                                        (oracle.WEIGHT, (1, 6)), (oracle.WEIGHT, (-2, -5)),
                                        (oracle.ACT, (2,)), (oracle.ACT, (-2,)), (oracle.ACT, (7,))]
                  for dtype in [torch.float32, torch.bfloat16, torch.float16]
                  if not (kind == oracle.ACT and dtype == torch.float32)]


@pytest.mark.parametrize("kind,offsets,dtype", _RESCALE_CASES)
def test_quantize_rescale_parity(kind, offsets, dtype):
    """RaZeR with rescaled large special values: bytes and tensor scale equal
    the oracle's, for both kinds and every input type."""
    _need_gpu()
    x = _rescale_input(kind, dtype, 17 + offsets[-1])
    ref = oracle.quantize(kind, as_f32(x), offsets, rescale=True)
    p = gpu_encode(kind, x, offsets, rescale=True)
    assert_same_encoding(p, ref, as_f32(x), f"rescale {kind} {offsets} {dtype}")


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("kind,offsets", [(oracle.WEIGHT, (-2, 4)), (oracle.ACT, (3,))])
def test_quantize_rescale_edge_cases(name, kind, offsets):
    _need_gpu()
    x = EDGE[name]
    ref = oracle.quantize(kind, x, offsets, rescale=True)
    p = gpu_encode(kind, torch.from_numpy(x), offsets, rescale=True)
    assert_same_encoding(p, ref, x, f"rescale edge {name} kind {kind}")


def test_quantize_rescale_prefill_weight_sampled():
    """The rescale mode on the full W[28672, 8192] fp32 weight with pairs
    (+-5, +-8): the oracle encodes a row sample with the row holding the tensor
    maximum (same tensor scale) and the GPU rows match it byte for byte."""
    _need_gpu()
    w = synth.prefill_weight()
    log("rescale prefill W: gpu ...")
    p = gpu_encode(oracle.WEIGHT, torch.from_numpy(w), (-2, 4), rescale=True)
    rmax = int(np.abs(w).max(axis=1).argmax())
    rows = sorted(set(np.random.default_rng(93).choice(w.shape[0], 96, replace=False).tolist()) | {rmax, 0, w.shape[0] - 1})
    log("rescale prefill W: oracle on", len(rows), "rows ...")
    ref = oracle.quantize_weight(w[rows], (-2, 4), rescale=True)
    k = w.shape[1]
    codes = p.codes.cpu().numpy().reshape(w.shape[0], k // 2)[rows]
    scales = p.scales.cpu().numpy().reshape(w.shape[0], k // 16)[rows]
    ts = p.tensor_scale.cpu().numpy().view(np.uint32)[0]
    assert ts == np.array([ref.tensor_scale], np.float32).view(np.uint32)[0]
    np.testing.assert_array_equal(scales.reshape(-1), ref.scales)
    np.testing.assert_array_equal(codes.reshape(-1), ref.codes)
    share8 = float(((scales >> 6) & 1).mean())
    log(f"rescale prefill W: blocks choosing +-8: {share8:.3f}")
    assert share8 > 0.1
    del p
    torch.cuda.empty_cache()


def test_rescaled_weights_decode_through_the_products():
    """A weight encoded with rescaled large special values goes through the
    GEMV, the small-batch product and the prefill tile kernel unchanged
    (decoding reads the scale byte and the metadata as for any RaZeR weight)."""
    _need_gpu()
    rng = np.random.default_rng(29)
    w = (rng.standard_t(5, (1040, 1024)) * 0.02).astype(np.float32)
    ref = oracle.quantize_weight(w, (-2, 4), rescale=True)
    p = rz.razer_quantize_weight(torch.from_numpy(w).cuda(), (-2, 4), rescale=True)
    for m in (1, 4, 16, 256):
        x = torch.from_numpy(rng.standard_normal((m, 1024)).astype(np.float32)).to(torch.bfloat16)
        y_ref, nrm = oracle.gemm(as_f32(x), ref)
        if m == 1:
            y = rz.razer_gemv(x.reshape(-1).to(torch.float16).cuda(), p, torch.float32).cpu().numpy()[None]
            y_ref, nrm = oracle.gemm(as_f32(x.to(torch.float16)), ref)
        else:
            y = rz.razer_gemm(x.cuda(), p, torch.float32).cpu().numpy()
        assert_product_close(y, y_ref, nrm, f"rescaled weight m={m}")


def test_four_over_six_weights_decode_through_the_products():
    # The Four Over Six layout is plain NVFP4, so the unchanged decoders
    # (dequant, GEMV, GEMM) read it exactly as the oracle's decoder does.
    _need_gpu()
    rng = np.random.default_rng(93)
    w = (rng.standard_t(5, (300, 512)) * 0.02).astype(np.float32)
    x = rng.standard_normal((5, 512)).astype(np.float32)
    ref = oracle.quantize_weight(w, (-2, 4), four_over_six=True)
    p = gpu_encode(oracle.WEIGHT, torch.from_numpy(w), (-2, 4), four_over_six=True)
    assert_same_encoding(p, ref, w, "4/6 weight")
    d = rz.razer_dequant(p, torch.float32).cpu().numpy()
    np.testing.assert_array_equal(d, oracle.dequant_f32(ref))
    xb = torch.from_numpy(x).to(torch.bfloat16)
    y_ref, nrm = oracle.gemm(as_f32(xb), ref)
    y = rz.razer_gemm(xb.cuda(), p, out_dtype=torch.float32).cpu().numpy()
    assert_product_close(y, y_ref, nrm, "4/6 gemm")
    y1 = rz.razer_gemv(xb[0].cuda(), p, out_dtype=torch.float32).cpu().numpy()
    assert_product_close(y1[None], y_ref[:1], nrm[:1], "4/6 gemv")


# ---- block-size and FP16 group-scale variants -------------------------------------

VARIANT_CASES = [  # kind, block, scale_fmt, mode, input dtype
    (oracle.WEIGHT, 32, 0, "razer", torch.float32), (oracle.WEIGHT, 64, 0, "razer", torch.bfloat16),
    (oracle.WEIGHT, 128, 0, "razer", torch.float16), (oracle.WEIGHT, 128, 1, "razer", torch.float32),
    (oracle.WEIGHT, 16, 1, "razer", torch.bfloat16), (oracle.WEIGHT, 64, 1, "razer", torch.float16),
    (oracle.ACT, 32, 0, "razer", torch.bfloat16), (oracle.ACT, 128, 0, "razer", torch.float16),
    (oracle.WEIGHT, 128, 0, "plain", torch.float32), (oracle.WEIGHT, 128, 1, "plain", torch.float32),
    (oracle.WEIGHT, 64, 0, "fos", torch.float32), (oracle.WEIGHT, 128, 1, "fos", torch.bfloat16),
    (oracle.ACT, 128, 0, "fos", torch.bfloat16), (oracle.ACT, 64, 0, "plain", torch.float16),
]


def _variant_encode(kind, x, offs, block, sfmt, mode):
    kw = dict(remap=mode != "plain", four_over_six=mode == "fos", block=block)
    ref = oracle.quantize(kind, as_f32(x), offs, scale_fmt=sfmt, **kw)
    xd = x.cuda()
    if kind == oracle.WEIGHT:
        p = rz.razer_quantize_weight(xd, offs, scale_fmt=sfmt, **kw)
    else:
        p = rz.razer_quantize_act(xd, offs, **kw)
    torch.cuda.synchronize()
    return p, ref


@pytest.mark.parametrize("kind,block,sfmt,mode,dtype", VARIANT_CASES)
def test_quantize_variant_parity(kind, block, sfmt, mode, dtype):
    _need_gpu()
    if kind == oracle.WEIGHT:
        x, offs = pr1()[0].to(dtype), (-2, -5)
    else:
        x, offs = synth.act_quant_x(64, 4096).to(dtype), (-2,)
    p, ref = _variant_encode(kind, x, offs, block, sfmt, mode)
    assert_same_encoding(p, ref, as_f32(x), f"variant kind {kind} block {block} fmt {sfmt} {mode} {dtype}")
    if mode == "razer":  # both candidates of every pair in use somewhere
        top = 15 if sfmt else 7
        sw = ref.scales.astype(np.int64)
        assert (sw >> top & 1).any() and (~sw >> top & 1).any()
    # the decoder reads the variant back exactly as the oracle's decoder does
    d32 = rz.razer_dequant(p, torch.float32).cpu().numpy()
    np.testing.assert_array_equal(d32, oracle.dequant_f32(ref))
    d16 = rz.razer_dequant(p, torch.bfloat16).cpu()
    assert torch.equal(d16, torch.from_numpy(oracle.dequant_f32(ref)).to(torch.bfloat16))


@pytest.mark.parametrize("name", [n for n in sorted(EDGE) if EDGE[n].shape[1] % 32 == 0])
@pytest.mark.parametrize("kind,block,sfmt", [(oracle.WEIGHT, 32, 1), (oracle.ACT, 32, 0), (oracle.WEIGHT, 32, 0)])
def test_quantize_variant_edge_cases(name, kind, block, sfmt):
    _need_gpu()
    x = EDGE[name]
    offs = (-2, -5) if kind == oracle.WEIGHT else (-2,)
    p, ref = _variant_encode(kind, torch.from_numpy(x), offs, block, sfmt, "razer")
    assert_same_encoding(p, ref, x, f"variant edge {name} kind {kind} block {block} fmt {sfmt}")
    if not np.isnan(ref.tensor_scale):
        np.testing.assert_array_equal(rz.razer_dequant(p, torch.float32).cpu().numpy(), oracle.dequant_f32(ref))


def test_quantize_variant_group128_f16_prefill_weight_sampled():
    """The pages' kernel layout (128-element blocks, FP16 scales with the
    metadata in the sign and top exponent bits) on the full W[28672, 8192]:
    rows sampled against the oracle with the tensor-maximum row included."""
    _need_gpu()
    w = synth.prefill_weight()
    log("g128 f16 prefill W: gpu ...")
    p = rz.razer_quantize_weight(torch.from_numpy(w).cuda(), (-2, 4), block=128, scale_fmt=rz.RAZER_SCALE_F16)
    torch.cuda.synchronize()
    rmax = int(np.abs(w).max(axis=1).argmax())
    rows = sorted(set(np.random.default_rng(97).choice(w.shape[0], 64, replace=False).tolist()) | {rmax})
    log("g128 f16 prefill W: oracle on", len(rows), "rows ...")
    ref = oracle.quantize(oracle.WEIGHT, w[rows], (-2, 4), block=128, scale_fmt=oracle.SCALE_F16)
    k = w.shape[1]
    codes = p.codes.cpu().numpy().reshape(w.shape[0], k // 2)[rows].reshape(-1)
    scales = p.scales.cpu().numpy().reshape(w.shape[0], -1)[rows].reshape(-1).view(np.uint16)
    assert p.tensor_scale.cpu().numpy().view(np.uint32)[0] == np.array([ref.tensor_scale], np.float32).view(np.uint32)[0]
    np.testing.assert_array_equal(scales, ref.scales)
    np.testing.assert_array_equal(codes, ref.codes)
    del p
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n,k,xdt", [(300, 1024, torch.float16), (77, 128, torch.bfloat16),
                                     (6144, 4096, torch.float16), (4096, 14336, torch.float16),
                                     (5, 65536, torch.bfloat16), (1000, 2944, torch.bfloat16),
                                     (1000, 8448, torch.bfloat16), (16, 12288, torch.float16)])
def test_gemv_group128_f16_layout(n, k, xdt):
    """The pages' kernel layout (128-element blocks, FP16 scales) through the
    GEMV: within tolerance of the fp64 product over the oracle's decoded
    weights; razer_gemm with m = 1 gives the same bytes.  Rows of more than
    8192 elements on up to 4096 rows (4096 x 14336, 1000 x 8448, 16 x 12288)
    go to the MFMA small-batch kernel."""
    _need_gpu()
    rng = np.random.default_rng(n + k)
    w = (rng.standard_t(5, (n, k)) * 0.02).astype(np.float32)
    ref = oracle.quantize(oracle.WEIGHT, w, (-2, -5), block=128, scale_fmt=oracle.SCALE_F16)
    x = torch.from_numpy(rng.standard_normal(k).astype(np.float32)).to(xdt)
    t = to_device(ref)
    y_ref, nrm = oracle.gemm_any(as_f32(x), ref)
    y32 = rz.razer_gemv(x.cuda(), t, torch.float32)
    y16 = rz.razer_gemv(x.cuda(), t, xdt)
    torch.cuda.synchronize()
    assert_product_close(y32.cpu().numpy()[None], y_ref, nrm, f"g128 gemv {n}x{k}")
    assert_product_close(y16.float().cpu().numpy()[None], y_ref, nrm, f"g128 gemv {n}x{k} 16-bit", xdt)
    assert torch.equal(rz.razer_gemm(x.cuda()[None], t, torch.float32)[0], y32)


def test_gemv_group_group128_f16_members():
    _need_gpu()
    rng = np.random.default_rng(141)
    refs = [oracle.quantize(oracle.WEIGHT, (rng.standard_t(5, (n, 2048)) * 0.02).astype(np.float32), offs,
                            block=128, scale_fmt=oracle.SCALE_F16)
            for n, offs in ((640, (-2, 4)), (96, (-2, -5)), (1, (-7, 7)))]
    ws = [to_device(r) for r in refs]
    x = torch.from_numpy(rng.standard_normal(2048).astype(np.float32)).to(torch.float16).cuda()
    ys = rz.razer_gemv_group(x, ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for r, wt, y in zip(refs, ws, ys):
        y_ref, nrm = oracle.gemm_any(x.float().cpu().numpy(), r)
        assert_product_close(y.cpu().numpy()[None], y_ref, nrm, "g128 group")
        assert torch.equal(y, rz.razer_gemv(x, wt, torch.float32))


def test_products_reject_variant_layouts():
    _need_gpu()
    w = rz.razer_quantize_weight(pr1()[0].cuda(), (-2, 4), block=64)
    x = torch.randn(1024, device="cuda", dtype=torch.float16)
    with pytest.raises(rz.RazerError) as e:
        rz.razer_gemv(x, w)
    assert e.value.status == rz.RAZER_E_UNSUPPORTED
    with pytest.raises(rz.RazerError):
        rz.razer_gemm(x.reshape(1, -1).repeat(4, 1), w)


# ---- decoder parity ------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("kind", [oracle.WEIGHT, oracle.ACT])
def test_dequant_parity(dtype, kind):
    _need_gpu()
    rng = np.random.default_rng(17)
    x = (rng.standard_t(4, (64, 272)) * 0.02).astype(np.float32)
    x[:, 5] *= 30
    offs = (-2, -5) if kind == oracle.WEIGHT else (-2,)
    ref = oracle.quantize(kind, x, offs)
    t = to_device(ref)
    out = rz.razer_dequant(t, dtype).cpu()
    want = torch.from_numpy(oracle.dequant_f32(ref)).to(dtype)  # RNE of the fp32 value
    assert torch.equal(out.view(torch.int16 if dtype != torch.float32 else torch.int32),
                       want.view(torch.int16 if dtype != torch.float32 else torch.int32))


# ---- product parity --------------------------------------------------------------

@pytest.mark.parametrize("out_dtype", [torch.float16, torch.float32])
def test_gemv_pr1(out_dtype):
    _need_gpu()
    w, x = pr1()
    ref = oracle.quantize_weight(w.numpy())
    y_ref, nrm = oracle.gemm(as_f32(x), ref)
    y = rz.razer_gemv(x.cuda().reshape(-1), to_device(ref), out_dtype).cpu().double().numpy()
    assert_product_close(y[None, :], y_ref, nrm, "gemv pr1", out_dtype)


@pytest.mark.parametrize("name", ["qkv", "gate", "up", "down"])
def test_gemv_llama3_8b_decode(name):
    _need_gpu()
    w = llama_weight(name)
    ref = llama_ref(name)
    x = synth.llama3_8b_decode_x(w.shape[1])
    log(f"gemv {name}: oracle product ...")
    y_ref, nrm = oracle.gemm(as_f32(x), ref)
    t = to_device(ref)
    y16 = rz.razer_gemv(x.cuda().reshape(-1), t, torch.float16).cpu().double().numpy()
    y32 = rz.razer_gemv(x.cuda().reshape(-1), t, torch.float32).cpu().double().numpy()
    e32 = assert_product_close(y32[None, :], y_ref, nrm, f"gemv {name} f32")
    e16 = assert_product_close(y16[None, :], y_ref, nrm, f"gemv {name} f16", torch.float16)
    log(f"gemv {name}: max err/norm f32 {e32:.2e} f16 {e16:.2e}")
    # the GPU encoder yields the same bytes for this weight
    p = gpu_encode(oracle.WEIGHT, torch.from_numpy(w), (-2, 4))
    assert_same_encoding(p, ref, None, f"llama {name} weight")


@pytest.mark.parametrize("n,k,xdt", [(7, 48, torch.float16), (33, 16, torch.bfloat16),
                                     (257, 1040, torch.float16), (64, 96, torch.bfloat16),
                                     (5, 65536, torch.float16), (3, 40976, torch.bfloat16),
                                     (9001, 2080, torch.float16)])
def test_gemv_ragged_shapes(n, k, xdt):
    _need_gpu()
    rng = np.random.default_rng(n * 7 + k)
    w = (rng.standard_t(5, (n, k)) * 0.02).astype(np.float32)
    x = torch.from_numpy(rng.normal(0, 1, k).astype(np.float32)).to(xdt)
    ref = oracle.quantize_weight(w, (-2, -5))
    y_ref, nrm = oracle.gemm(as_f32(x)[None, :], ref)
    y = rz.razer_gemv(x.cuda(), to_device(ref), torch.float32).cpu().double().numpy()
    assert_product_close(y[None, :], y_ref, nrm, f"gemv {n}x{k}")


def test_gemv_group_llama3_8b_gate_up():
    """Gate and up of the decode layer in one launch: each output within
    tolerance of the oracle and bitwise equal to its own razer_gemv."""
    _need_gpu()
    x = synth.llama3_8b_decode_x(4096).reshape(-1)
    ref = {n: llama_ref(n) for n in ("gate", "up")}
    ws = [to_device(ref["gate"]), to_device(ref["up"])]
    xd = x.cuda()
    ys = rz.razer_gemv_group(xd, ws)
    torch.cuda.synchronize()
    for n, w, y in zip(("gate", "up"), ws, ys):
        y_ref, nrm = oracle.gemm(as_f32(x), ref[n])
        assert_product_close(y.float().cpu().numpy()[None], y_ref, nrm, f"group {n}", torch.float16)
        assert torch.equal(y, rz.razer_gemv(xd, w)), n


@pytest.mark.parametrize("xdt", [torch.float16, torch.bfloat16])
def test_gemv_group_ragged_members(xdt):
    # four members with different rows (one empty, one a single row), both
    # kinds, different offsets and tensor scales; a member with K > 8192 on
    # few rows takes the small-batch kernel on its own
    _need_gpu()
    rng = np.random.default_rng(111)
    for k in (1040, 16384):
        shapes = [(300, (-2, 4), oracle.WEIGHT), (0, (-2, 4), oracle.WEIGHT), (1, (-7, 7), oracle.WEIGHT),
                  (77, (-2,), oracle.ACT)]
        refs, ws = [], []
        for i, (n, offs, kind) in enumerate(shapes):
            w = (rng.standard_t(5, (n, k)) * 0.02 * (i + 1)).astype(np.float32)
            r = oracle.quantize(kind, w, offs)
            refs.append(r)
            ws.append(to_device(r))
        x = torch.from_numpy(rng.standard_normal(k).astype(np.float32)).to(xdt)
        ys = rz.razer_gemv_group(x.cuda(), ws, out_dtype=torch.float32)
        torch.cuda.synchronize()
        for i, (r, w, y) in enumerate(zip(refs, ws, ys)):
            assert y.shape == (r.rows,)
            if r.rows == 0:
                continue
            y_ref, nrm = oracle.gemm(as_f32(x), r)
            assert_product_close(y.cpu().numpy()[None], y_ref, nrm, f"group member {i} k {k}")
            assert torch.equal(y, rz.razer_gemv(x.cuda(), w, out_dtype=torch.float32)), (i, k)


def test_gemv_nan_tensor_scale_gives_nan():
    _need_gpu()
    x = EDGE["nan"]
    ref = oracle.quantize_weight(x, (-2, 4))
    t = to_device(ref)
    y = rz.razer_gemv(torch.ones(64, dtype=torch.float16, device="cuda"), t, torch.float32).cpu()
    assert torch.isnan(y).all()


@pytest.mark.parametrize("m", [2, 3, 4, 8, 16, 32])
def test_gemm_small_batch_4096(m):
    _need_gpu()
    ref = small_batch_ref(4096, 4096)
    x32 = synth.small_batch_x(32, 4096)
    y_ref, nrm = _small_batch_oracle_4096()
    t = to_device(ref)
    x = synth.small_batch_x(m, 4096).cuda()
    y = rz.razer_gemm(x, t, torch.float32).cpu().double().numpy()
    assert torch.equal(x.cpu(), x32[:m])
    e = assert_product_close(y, y_ref[:m], nrm[:m], f"gemm m={m} 4096x4096")
    log(f"gemm m={m} 4096: max err/norm {e:.2e}")


@functools.lru_cache(maxsize=None)
def _small_batch_oracle_4096():
    log("gemm 4096: oracle product for M=32 ...")
    return oracle.gemm(as_f32(synth.small_batch_x(32, 4096)), small_batch_ref(4096, 4096))


@pytest.mark.parametrize("m", [2, 3, 4, 6, 8, 32])
def test_gemm_small_batch_70b_sampled(m):
    _need_gpu()
    log("gemm 70b: reference encode ...")
    ref = small_batch_ref(28672, 8192)
    t = to_device(ref)
    x = synth.small_batch_x(m, 8192)
    y = rz.razer_gemm(x.cuda(), t, torch.bfloat16).cpu().double().numpy()
    cols = np.random.default_rng(m).choice(28672, 256, replace=False)
    y_ref, nrm = oracle.gemm(as_f32(x), ref, cols)
    assert_product_close(y[:, cols], y_ref, nrm, f"gemm m={m} 28672x8192 (256 sampled columns)",
                         torch.bfloat16)


def test_gemm_prefill_sampled():
    """Prefill product M=2048, N=28672, K=8192 (bf16), checked on sampled columns."""
    _need_gpu()
    ref = _prefill_weight_packed()
    t = to_device(ref)
    x = synth.prefill_x()
    log("prefill: gpu gemm ...")
    y = rz.razer_gemm(x.cuda(), t, torch.bfloat16)
    torch.cuda.synchronize()
    cols = np.random.default_rng(2048).choice(28672, 24, replace=False)
    yc = y[:, torch.from_numpy(cols).cuda()].cpu().double().numpy()
    log("prefill: oracle product on 24 columns ...")
    y_ref, nrm = oracle.gemm(as_f32(x), ref, cols)
    e = assert_product_close(yc, y_ref, nrm, "prefill gemm (24 sampled columns x 2048 rows)",
                             torch.bfloat16)
    log(f"prefill: max err/norm {e:.2e}")
    # every output is finite
    assert torch.isfinite(y).all()


@pytest.mark.parametrize("m,n,k,xdt", [(3, 100, 48, torch.bfloat16), (130, 257, 80, torch.float16),
                                       (2, 16, 16, torch.bfloat16), (129, 129, 4096, torch.bfloat16),
                                       (33, 64, 32, torch.float16), (257, 300, 128, torch.bfloat16),
                                       (512, 256, 192, torch.float16), (300, 520, 4096, torch.bfloat16),
                                       (3, 33, 320, torch.float16), (2, 50, 384, torch.bfloat16),
                                       (4, 1000, 4096, torch.float16), (2, 17, 256, torch.float16),
                                       (3, 64, 960, torch.bfloat16), (2, 40, 320, torch.bfloat16),
                                       (5, 100, 512, torch.bfloat16), (17, 77, 768, torch.float16),
                                       (32, 4100, 1024, torch.bfloat16), (9, 16, 256, torch.float16)])
def test_gemm_ragged_shapes(m, n, k, xdt):
    _need_gpu()
    rng = np.random.default_rng(m * 1000 + n + k)
    w = (rng.standard_t(4, (n, k)) * 0.015).astype(np.float32)
    x = torch.from_numpy(rng.normal(0, 1, (m, k)).astype(np.float32)).to(xdt)
    ref = oracle.quantize_weight(w, (-2, -5))
    y_ref, nrm = oracle.gemm(as_f32(x), ref)
    for odt in (torch.float32, torch.bfloat16):
        y = rz.razer_gemm(x.cuda(), to_device(ref), odt).cpu().double().numpy()
        assert_product_close(y, y_ref, nrm, f"gemm {m}x{n}x{k} out {odt}", odt)


@pytest.mark.parametrize("m", [3, 5, 6, 7, 8])
def test_gemm_three_to_eight_rows(m):
    """Three to eight rows on K % 256 == 0: every row count, weight rows that
    leave part of the last 64-row workgroup empty, one-unit and split K, both
    input types, checked element by element against the oracle."""
    _need_gpu()
    for n, k, xdt in [(200, 768, torch.bfloat16), (64, 256, torch.float16), (1000, 4096, torch.bfloat16),
                      (17, 2048, torch.float16)]:
        rng = np.random.default_rng(m * 7919 + n + k)
        w = (rng.standard_t(4, (n, k)) * 0.015).astype(np.float32)
        x = torch.from_numpy(rng.normal(0, 1, (m, k)).astype(np.float32)).to(xdt)
        ref = oracle.quantize_weight(w, (-2, 4))
        y_ref, nrm = oracle.gemm(as_f32(x), ref)
        for odt in (torch.float32, torch.float16):
            y = rz.razer_gemm(x.cuda(), to_device(ref), odt).cpu().double().numpy()
            assert_product_close(y, y_ref, nrm, f"gemm {m}x{n}x{k} out {odt}", odt)


@pytest.mark.parametrize("m,n,k", [(1, 200, 1024), (1, 5000, 512), (2, 96, 768), (4, 40, 512),
                                   (8, 64, 512), (300, 260, 256)])
def test_products_with_activation_kind_operand(m, n, k):
    """The products take a packed tensor of either kind: an E4M3 / 1-bit
    activation encoding used as the right operand goes through every product
    kernel (GEMV, small batch, batch, prefill) against the oracle."""
    _need_gpu()
    rng = np.random.default_rng(n * 31 + k + m)
    w = rng.normal(0, 1, (n, k)).astype(np.float32)
    w[:, rng.choice(k, 4, replace=False)] *= 20.0
    ref = oracle.quantize_act(w, (-2,))
    x = torch.from_numpy(rng.normal(0, 1, (m, k)).astype(np.float32)).to(torch.bfloat16)
    y_ref, nrm = oracle.gemm(as_f32(x), ref)
    t = to_device(ref)
    if m == 1:
        y = rz.razer_gemv(x.cuda().reshape(-1), t, torch.float32).cpu().double().numpy()[None, :]
    else:
        y = rz.razer_gemm(x.cuda(), t, torch.float32).cpu().double().numpy()
    assert_product_close(y, y_ref, nrm, f"act-kind operand {m}x{n}x{k}")


# ---- second-pair offset search (offline weight encoder) ---------------------------

@functools.lru_cache(maxsize=1)
def _offset_cases():
    rng = np.random.default_rng(23)
    t = (rng.standard_t(5, (64, 256)) * 0.02).astype(np.float32)
    t[:, 9] *= 15
    planted = np.zeros((4, 64), np.float32)  # every block: 6.0 and 3.5 (best offset -5)
    planted[:, 0::16] = 6.0
    planted[:, 5::16] = 3.5
    ragged = (rng.standard_normal((3, 48)) * 0.1).astype(np.float32)
    # blocks ~1/1000 of the tensor maximum get subnormal E3M3 scale codes, so
    # scaled values reach up to 9 and the second pairs above 6 can move them
    sub = (rng.standard_normal((8, 64)) * 0.01).astype(np.float32)
    sub[0, 0] = 30.0
    nan = t[:2].copy()
    nan[1, 3] = np.nan
    return {"student_t": t, "planted": planted, "ragged": ragged, "subnormal_scales": sub,
            "zeros": np.zeros((2, 32), np.float32), "empty": np.zeros((0, 32), np.float32),
            "nonfinite": nan}


def _check_offset_sse(got, ref, what):
    assert np.array_equal(np.isnan(got), np.isnan(ref)), what
    ok = ~np.isnan(ref)
    np.testing.assert_allclose(got[ok], ref[ok], rtol=1e-9, atol=1e-300, err_msg=what)
    if ok.all() and ref.size:
        # the offset the oracle picks is also a minimum of the GPU's sums
        assert got[int(np.argmin(ref))] <= got.min() * (1 + 1e-9), what


@pytest.mark.parametrize("name", sorted(_offset_cases()))
@pytest.mark.parametrize("off0", [-2, 3])
def test_offset_sse_matches_oracle(name, off0):
    _need_gpu()
    w = _offset_cases()[name]
    ref = oracle.weight_offset_sse(w, off0)
    got = rz.razer_weight_offset_sse(torch.from_numpy(w).cuda(), off0).cpu().numpy()
    _check_offset_sse(got, ref, f"{name} off0={off0}")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_offset_sse_16bit_inputs(dtype):
    _need_gpu()
    w16 = torch.from_numpy(_offset_cases()["student_t"]).to(dtype)
    ref = oracle.weight_offset_sse(w16.float().numpy(), -2)
    got = rz.razer_weight_offset_sse(w16.cuda(), -2).cpu().numpy()
    _check_offset_sse(got, ref, str(dtype))


def test_offset_sse_planted_and_best_offset():
    _need_gpu()
    best, sse = rz.razer_best_second_offset(torch.from_numpy(_offset_cases()["planted"]).cuda(), -2)
    assert best == -5
    assert sse[best + 7] < 1e-9


def test_offset_sse_full_size_prefill_weight():
    """W[28672, 8192] fp32 ~ 0.015 t(4): the default offset's sum against the
    oracle, the exact equalities that hold at any size, repeatability."""
    _need_gpu()
    log("offset search: generating ...")
    w = synth.prefill_weight()
    wd = torch.from_numpy(w).cuda()
    log("offset search: gpu ...")
    got = rz.razer_weight_offset_sse(wd, -2).cpu().numpy()
    again = rz.razer_weight_offset_sse(wd, -2).cpu().numpy()
    assert np.array_equal(got.view(np.uint64), again.view(np.uint64))
    # a second pair on the FP4 grid (M = 3, 4, 6) moves nothing, exactly like
    # a second pair equal to the first: same encodings, same summation order
    for o in (-6, -4, 0):
        assert got[o + 7] == got[-2 + 7]
    log("offset search: oracle at offset +4 ...")
    d = oracle.dequant_f64(oracle.quantize_weight(w, (-2, 4)))
    ref4 = float(np.sum((w.astype(np.float64) - d) ** 2))
    del d
    assert abs(got[4 + 7] - ref4) <= 1e-9 * ref4
    del wd
    torch.cuda.empty_cache()


# ---- W4A4 product ------------------------------------------------------------------

W4A4_CASES = [(1, 512, 1024, torch.float32), (1, 4096, 14336, torch.float16), (3, 100, 48, torch.bfloat16),
              (8, 4096, 4096, torch.bfloat16), (32, 1000, 512, torch.float32), (256, 512, 1024, torch.bfloat16),
              (300, 130, 272, torch.float16),
              # prefill shapes whose product applies both tensor scales in its epilogue
              (512, 200, 640, torch.float32), (260, 96, 128, torch.float16)]


def _w4a4_operands(m, n, k, x_kind=oracle.ACT, x_offsets=(-2,)):
    rng = np.random.default_rng(m * 7919 + n * 31 + k)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, 3] *= 20  # an outlier channel
    w = (rng.standard_t(5, (n, k)) * 0.02).astype(np.float32)
    return oracle.quantize(x_kind, x, x_offsets), oracle.quantize_weight(w, (-2, 4))


@pytest.mark.parametrize("m,n,k,ydt", W4A4_CASES)
def test_gemm_w4a4_matches_oracle(m, n, k, ydt):
    _need_gpu()
    log(f"w4a4 {m}x{n}x{k} {ydt}")
    xp, wp = _w4a4_operands(m, n, k)
    y = rz.razer_gemm_w4a4(to_device(xp), to_device(wp), ydt).cpu().double().numpy()
    y_ref, nrm = oracle.gemm_w4a4(xp, wp)
    assert_product_close(y, y_ref, nrm, f"w4a4 {m}x{n}x{k}", ydt)


def test_gemm_w4a4_weight_kind_left_operand():
    # a left operand with the weight encoding and offsets (-7, 7): special
    # values +/-2.5 and +/-9.5 times E3M3 scales need 9 significant bits
    _need_gpu()
    xp, wp = _w4a4_operands(16, 96, 256, oracle.WEIGHT, (-7, 7))
    y = rz.razer_gemm_w4a4(to_device(xp), to_device(wp), torch.float32).cpu().double().numpy()
    y_ref, nrm = oracle.gemm_w4a4(xp, wp)
    assert_product_close(y, y_ref, nrm, "w4a4 weight-kind x", torch.float32)


def test_gemm_w4a4_prefill_sampled():
    """W4A4 at the prefill shape M=2048, N=28672, K=8192, on sampled columns."""
    _need_gpu()
    wp = _prefill_weight_packed()
    log("w4a4 prefill: oracle act encode ...")
    xp = oracle.quantize_act(synth.prefill_x().float().numpy(), (-2,))
    log("w4a4 prefill: gpu ...")
    y = rz.razer_gemm_w4a4(to_device(xp), to_device(wp), torch.bfloat16)
    torch.cuda.synchronize()
    cols = np.random.default_rng(4404).choice(28672, 16, replace=False)
    yc = y[:, torch.from_numpy(cols).cuda()].cpu().double().numpy()
    log("w4a4 prefill: oracle product on 16 columns ...")
    y_ref, nrm = oracle.gemm_w4a4(xp, wp, cols)
    assert_product_close(yc, y_ref, nrm, "w4a4 prefill (16 sampled columns x 2048 rows)", torch.bfloat16)
    assert torch.isfinite(y).all()


# ---- graph capture ---------------------------------------------------------------

def test_graph_replays_match_eager_results():
    """Every call enqueues kernels only (no allocation, no memset, no host
    sync), so a captured sequence replays the eager results bit for bit; each
    of three replays is checked, with eager work in between."""
    _need_gpu()
    rng = np.random.default_rng(121)
    dev = "cuda"
    w_np = (rng.standard_t(5, (512, 1024)) * 0.02).astype(np.float32)
    w = torch.from_numpy(w_np).to(dev)
    xa = torch.from_numpy(rng.standard_normal((300, 1024)).astype(np.float32)).to(dev).to(torch.bfloat16)
    x1 = xa[0].to(torch.float16).contiguous()
    xs = xa[:8].contiguous()
    wq = rz.razer_quantize_weight(w, (-2, 4))
    w2 = rz.razer_quantize_weight(w[:300].contiguous(), (-2, -5))
    outs = {
        "act": rz.PackedTensor(rz.RAZER_ACT, 300, 1024, (-2,), dev),
        "wenc": rz.PackedTensor(rz.RAZER_WEIGHT, 512, 1024, (-2, 4), dev),
        "gemv": torch.empty(512, dtype=torch.float16, device=dev),
        "g0": torch.empty(512, dtype=torch.float16, device=dev),
        "g1": torch.empty(300, dtype=torch.float16, device=dev),
        "small": torch.empty((8, 512), dtype=torch.bfloat16, device=dev),
        "prefill": torch.empty((300, 512), dtype=torch.bfloat16, device=dev),
        "deq": torch.empty((512, 1024), dtype=torch.bfloat16, device=dev),
    }
    wsa = torch.empty(max(1, rz.razer_workspace_bytes(rz.RAZER_OP_QUANTIZE_ACT, 300, 0, 1024)),
                      dtype=torch.uint8, device=dev)
    wsw = torch.empty(max(1, rz.razer_workspace_bytes(rz.RAZER_OP_QUANTIZE_WEIGHT, 512, 0, 1024)),
                      dtype=torch.uint8, device=dev)
    wss = torch.empty(max(1, rz.razer_workspace_bytes(rz.RAZER_OP_GEMM, 8, 512, 1024)),
                      dtype=torch.uint8, device=dev)

    def seq():
        rz.razer_quantize_act(xa, out=outs["act"], workspace=wsa)
        rz.razer_quantize_weight(w, out=outs["wenc"], workspace=wsw)
        rz.razer_gemv(x1, wq, out=outs["gemv"])
        rz.razer_gemv_group(x1, [wq, w2], outs=[outs["g0"], outs["g1"]])
        rz.razer_gemm(xs, wq, out=outs["small"], workspace=wss)
        rz.razer_gemm(xa, wq, out=outs["prefill"])
        rz.razer_dequant(wq, out=outs["deq"])

    def snapshot():
        snap = {}
        for key, v in outs.items():
            if isinstance(v, rz.PackedTensor):
                snap[key] = (v.codes.clone(), v.scales.clone(), v.tensor_scale.clone())
            else:
                snap[key] = (v.clone(),)
        return snap

    def clear():
        for v in outs.values():
            for t in ((v.codes, v.scales, v.tensor_scale) if isinstance(v, rz.PackedTensor) else (v,)):
                t.zero_()

    seq()
    torch.cuda.synchronize()
    ref = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    for rep in range(3):
        clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for key in ref:
            for a, b in zip(ref[key], got[key]):
                assert torch.equal(a, b), f"replay {rep}: {key} differs"
        rz.razer_gemv(x1, wq, out=torch.empty(512, dtype=torch.float16, device=dev))  # eager work between
        torch.cuda.synchronize()
