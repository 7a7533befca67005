"""The Python binding checks caller-supplied outputs, workspaces and packed
tensors before it calls the C ABI, which cannot see buffer sizes: a wrong
shape, dtype, device or layout raises, and nothing is enqueued (the output's
sentinel values survive a synchronize)."""
import pytest
import torch

import nvfp4_razer_w4a16_amd as rz


def test_cpu_tensors_are_rejected_before_any_call():
    # host memory handed to a device kernel would fault: every entry point
    # refuses it (these checks run without a GPU)
    w = rz.PackedTensor(rz.RAZER_WEIGHT, 64, 256, (-2, 4), "cpu")
    x = torch.zeros(256, dtype=torch.float16)
    for call in (lambda: rz.razer_gemv(x, w), lambda: rz.razer_gemm(x.reshape(1, -1), w),
                 lambda: rz.razer_dequant(w), lambda: rz.razer_gemv_group(x, [w]),
                 lambda: rz.razer_quantize_weight(torch.zeros(64, 256)),
                 lambda: rz.razer_quantize_act(torch.zeros(64, 256, dtype=torch.bfloat16)),
                 lambda: rz.razer_gemm_w4a4(w, w),
                 lambda: rz.razer_weight_offset_sse(torch.zeros(64, 256))):
        with pytest.raises(ValueError, match="must be on"):
            call()


def test_packed_tensor_with_replaced_buffers_is_rejected():
    w = rz.PackedTensor(rz.RAZER_WEIGHT, 64, 256, (-2, 4), "cpu")
    w.codes = torch.zeros(64, 64, dtype=torch.uint8)  # half the bytes
    with pytest.raises(ValueError, match="codes has shape"):
        w.check()
    w = rz.PackedTensor(rz.RAZER_WEIGHT, 64, 256, (-2, 4), "cpu")
    w.tensor_scale = torch.zeros(1, dtype=torch.float64)
    with pytest.raises(ValueError, match="tensor_scale has dtype"):
        w.check()


def _sentinel(shape, dtype, dev):
    return torch.full(shape, 7.0, dtype=dtype, device=dev)


@pytest.mark.gpu
def test_mismatched_outputs_raise_and_enqueue_nothing():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(3)
    wf = (torch.randn(96, 512, generator=g) * 0.02).to(dev)
    w = rz.razer_quantize_weight(wf)
    w2 = rz.razer_quantize_weight(wf[:64].contiguous())
    x = torch.randn(512, generator=g).to(torch.float16).to(dev)
    torch.cuda.synchronize()
    cases = []
    y = _sentinel((95,), torch.float32, dev)  # one element short
    cases.append((lambda y=y: rz.razer_gemv(x, w, out=y), y))
    y = _sentinel((96, 2), torch.float32, dev)[:, 0]  # not contiguous
    cases.append((lambda y=y: rz.razer_gemv(x, w, out=y), y))
    y = _sentinel((96,), torch.float64, dev)  # unsupported dtype
    cases.append((lambda y=y: rz.razer_gemv(x, w, out=y), y))
    ya, yb = _sentinel((96,), torch.float32, dev), _sentinel((64,), torch.float16, dev)  # mixed dtypes
    cases.append((lambda ya=ya, yb=yb: rz.razer_gemv_group(x, [w, w2], outs=[ya, yb]), ya))
    ya, yb = _sentinel((96,), torch.float32, dev), _sentinel((96,), torch.float32, dev)  # second too big
    cases.append((lambda ya=ya, yb=yb: rz.razer_gemv_group(x, [w, w2], outs=[ya, yb]), ya))
    xm = torch.randn(4, 512, generator=g).to(torch.bfloat16).to(dev)
    y = _sentinel((4, 95), torch.float32, dev)
    cases.append((lambda y=y: rz.razer_gemm(xm, w, out=y), y))
    y = _sentinel((96, 256), torch.float32, dev)
    cases.append((lambda y=y: rz.razer_dequant(w, out=y), y))
    # an encoder output larger than the input: its loads would run past x
    big = rz.PackedTensor(rz.RAZER_WEIGHT, 128, 512, (-2, 4), dev)
    big.codes.fill_(0x55)
    cases.append((lambda: rz.razer_quantize_weight(wf, out=big), big.codes))
    y = _sentinel((15,), torch.float32, dev)
    cases.append((lambda y=y: rz.razer_weight_offset_sse(wf, out=y), y))
    xq = rz.razer_quantize_act(xm)
    y = _sentinel((4, 97), torch.float32, dev)
    cases.append((lambda y=y: rz.razer_gemm_w4a4(xq, w, out=y), y))
    torch.cuda.synchronize()
    for i, (call, buf) in enumerate(cases):
        before = buf.clone()
        with pytest.raises(ValueError):
            call()
        torch.cuda.synchronize()
        assert torch.equal(buf, before), f"case {i} wrote its output"
