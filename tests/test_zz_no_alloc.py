"""razer_quantize_act_noalloc (the allocation-free activation encoder) through
the C ABI: bit-identical to razer_quantize_act on the same input, on two calls
in a row, the second with a smaller input (the static scratch keeps the first
call's partials, which the second must not read)."""
import ctypes

import numpy as np
import pytest
import torch

import nvfp4_razer_w4a16_amd as rz

pytestmark = pytest.mark.gpu


def _noalloc(x: torch.Tensor, out: rz.PackedTensor) -> int:
    L = rz.lib()
    f = L.razer_quantize_act_noalloc
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(rz.razer_packed), ctypes.c_void_p]
    s = out.struct()
    return f(ctypes.c_void_p(x.data_ptr()), rz._dtype_code(x.dtype), ctypes.byref(s),
             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _input(rows, cols, seed, scale, dtype):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(rows, cols, generator=g) * scale
    x[:, 7] *= 40.0  # an outlier channel
    return x.to(dtype).cuda()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_noalloc_matches_workspace_encoder_on_two_calls(dtype):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # the first input is large (every amax partial written), the second small
    # with a much smaller maximum: a stale partial would change its tensor scale
    for rows, cols, seed, scale in ((4096, 8192, 1, 1.0), (33, 160, 2, 1e-3)):
        x = _input(rows, cols, seed, scale, dtype)
        ref = rz.razer_quantize_act(x)
        got = rz.PackedTensor(rz.RAZER_ACT, rows, cols, (-2,), x.device)
        got.codes.fill_(0xAA)
        got.scales.fill_(0xAA)
        assert _noalloc(x, got) == rz.RAZER_OK
        torch.cuda.synchronize()
        assert torch.equal(got.tensor_scale, ref.tensor_scale), (rows, cols)
        assert torch.equal(got.codes, ref.codes), (rows, cols)
        assert torch.equal(got.scales, ref.scales), (rows, cols)
        assert np.isfinite(float(got.tensor_scale.cpu()[0]))


def test_noalloc_rejects_what_the_workspace_encoder_rejects():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    x = _input(8, 64, 3, 1.0, torch.bfloat16)
    w = rz.PackedTensor(rz.RAZER_WEIGHT, 8, 64, (-2, 4), x.device)  # wrong kind
    assert _noalloc(x, w) == rz.RAZER_E_INVALID
    a = rz.PackedTensor(rz.RAZER_ACT, 8, 64, (-2,), x.device)
    a.offsets = (9,)  # outside [-7, 7]
    assert _noalloc(x, a) == rz.RAZER_E_INVALID
