"""Helpers shared by the GPU test modules: seeded workloads (cached), the
oracle's packed tensors uploaded to the device, and the comparisons (bit-exact
encodings; products within 2e-3 * sum |x||w| per output).  No expected value
comes from the GPU path."""
import functools
import sys

import numpy as np
import pytest
import torch

import nvfp4_razer_w4a16_amd as rz
import oracle
from nvfp4_razer_w4a16_amd import synth

TOL = 2e-3  # relative to sum |x||w| per output

# Rounding the finished fp32 value to a 16-bit output adds up to half an ulp
# of that format on top of the product tolerance (bf16: 8 significant bits,
# fp16: 11).  With small K, |y| comes close to sum |x||w| and this term alone
# can exceed 2e-3 * sum |x||w|.
OUT_MANT_BITS = {None: None, "float32": None, "float16": 11, "bfloat16": 8}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ---- helpers -----------------------------------------------------------------

def gpu_encode(kind, x_cpu: torch.Tensor, offsets, remap=True, four_over_six=False, rescale=False):
    x = x_cpu.cuda()
    if kind == oracle.WEIGHT:
        p = rz.razer_quantize_weight(x, offsets, remap, four_over_six=four_over_six, rescale=rescale)
    else:
        p = rz.razer_quantize_act(x, offsets, remap, four_over_six=four_over_six, rescale=rescale)
    torch.cuda.synchronize()
    return p


def as_f32(x_cpu: torch.Tensor) -> np.ndarray:
    return x_cpu.float().numpy()


def assert_same_encoding(p: rz.PackedTensor, ref: oracle.Packed, x=None, what=""):
    codes = p.codes.cpu().numpy().reshape(-1)
    scales = p.scales.cpu().numpy().reshape(-1).view(ref.scales.dtype)  # 2-byte FP16 scales
    ts = p.tensor_scale.cpu().numpy().view(np.uint32)[0]
    ts_ref = np.array([ref.tensor_scale], dtype=np.float32).view(np.uint32)[0]
    assert ts == ts_ref, f"{what}: tensor scale {ts:#x} vs {ts_ref:#x}"
    bad_s = np.nonzero(scales != ref.scales)[0]
    bad_c = np.nonzero(codes != ref.codes)[0]
    if bad_s.size or bad_c.size:
        B = getattr(ref, "block", 16)
        blk = int(bad_s[0]) if bad_s.size else int(bad_c[0]) // (B // 2)
        cb = slice(B // 2 * blk, B // 2 * blk + min(B // 2, 16))
        msg = (f"{what}: {bad_s.size} scales and {bad_c.size} code bytes differ; first block {blk}: "
               f"gpu scale {int(scales[blk]):#06x} codes {codes[cb].tolist()} / "
               f"ref scale {int(ref.scales[blk]):#06x} codes {ref.codes[cb].tolist()}")
        if x is not None:
            msg += f"; block input {np.asarray(x).reshape(-1)[B*blk:B*blk+min(B, 32)].tolist()}"
        raise AssertionError(msg)


def to_device(pk: oracle.Packed) -> rz.PackedTensor:
    t = rz.PackedTensor(pk.kind, pk.rows, pk.cols, pk.offsets, "cuda", 0, pk.block, pk.scale_fmt)
    t.codes.copy_(torch.from_numpy(pk.codes.reshape(pk.rows, pk.cols // 2)))
    t.scales.copy_(torch.from_numpy(pk.scales.view(np.uint8).reshape(tuple(t.scales.shape))))
    t.tensor_scale.copy_(torch.tensor([float(pk.tensor_scale)], dtype=torch.float32))
    return t


def assert_product_close(y_gpu: np.ndarray, y_ref: np.ndarray, norm: np.ndarray, what="",
                         out_dtype=None):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    bound = TOL * norm
    bits = OUT_MANT_BITS[str(out_dtype).replace("torch.", "") if out_dtype is not None else None]
    if bits is not None:
        mag = np.maximum(np.abs(y_ref), np.abs(y_gpu))
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
        bound = bound + np.where(mag > 0, np.ldexp(0.5, (e - (bits - 1)).astype(np.int64)), 0.0)
    bad = ~((err <= bound) | ((norm == 0) & (y_gpu == 0)))
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(bound, 1e-300), 0)), bad.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs out of tolerance; worst at "
                             f"{i}: gpu {y_gpu[i]!r} ref {y_ref[i]!r} norm {norm[i]!r}")
    return float((err / np.maximum(norm, 1e-300)).max())


# ---- cached workloads ----------------------------------------------------------

@functools.lru_cache(maxsize=None)
def pr1():
    w, x = synth.pr1_tiny()
    return torch.from_numpy(w), x


@functools.lru_cache(maxsize=None)
def llama_weight(name):
    return synth.llama3_8b_decode_weight(name)


@functools.lru_cache(maxsize=None)
def llama_ref(name):
    return oracle.quantize_weight(llama_weight(name))


@functools.lru_cache(maxsize=None)
def small_batch_ref(n, k):
    w = synth.small_batch_weight(n, k)
    ref = oracle.quantize_weight(w, (-2, 4))
    return ref


@functools.lru_cache(maxsize=1)
def prefill_weight_packed() -> oracle.Packed:
    log("prefill: generating W ...")
    w = synth.prefill_weight()
    log("prefill: oracle encode ...")
    return oracle.quantize_weight(w, (-2, 4))
