"""RaZeR-NVFP4 W4A16 on AMD MI355X (gfx950): Python binding of librazer.

Thin ctypes marshalling over the C ABI in ``include/librazer.h``; every step of
the computation runs in librazer's HIP kernels.  PyTorch supplies device memory
(outputs and workspaces are torch tensors) and the current HIP stream.  If
``librazer.so`` has not been built, every call raises ``RuntimeError``: there is
no fallback path.

Functions carry the C names: ``razer_quantize_weight``, ``razer_quantize_act``,
``razer_dequant``, ``razer_gemv``, ``razer_gemm``, ``razer_gemm_w4a4``, ``razer_weight_offset_sse``,
``razer_workspace_bytes``, ``razer_status_string``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librazer.so")

RAZER_OK, RAZER_E_INVALID, RAZER_E_UNSUPPORTED, RAZER_E_HIP = 0, 1, 2, 3
RAZER_F32, RAZER_F16, RAZER_BF16 = 0, 1, 2
RAZER_WEIGHT, RAZER_ACT = 0, 1
RAZER_FLAG_NO_REMAP, RAZER_FLAG_FOUR_OVER_SIX, RAZER_FLAG_UNTRIMMED_PLAN, RAZER_FLAG_RESCALE_LARGE_SV = 1, 2, 4, 8
RAZER_SCALE_BYTE, RAZER_SCALE_F16 = 0, 1
BLOCK_SIZES = (16, 32, 64, 128)
RAZER_OP_QUANTIZE_WEIGHT, RAZER_OP_QUANTIZE_ACT, RAZER_OP_GEMV, RAZER_OP_GEMM = 0, 1, 2, 3
RAZER_OP_OFFSET_SEARCH, RAZER_OP_GEMM_W4A4, RAZER_OP_GEMM_UNTRIMMED = 4, 5, 6
SECOND_PAIR_OFFSETS = tuple(range(-7, 8))  # entry i of razer_weight_offset_sse is offset i - 7

EXPORTED = ("razer_quantize_weight", "razer_quantize_act", "razer_quantize_act_noalloc", "razer_dequant", "razer_gemv",
            "razer_gemv_group", "razer_gemm", "razer_gemm_w4a4", "razer_weight_offset_sse", "razer_workspace_bytes",
            "razer_status_string")

DEFAULT_WEIGHT_OFFSETS = (-2, 4)  # special values +/-5 and +/-8
DEFAULT_ACT_OFFSETS = (-2,)       # special values +/-5

_DT = {torch.float32: RAZER_F32, torch.float16: RAZER_F16, torch.bfloat16: RAZER_BF16}


class razer_packed(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("flags", ctypes.c_uint32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("sv_off_half", ctypes.c_int8 * 2),
                ("block_log2", ctypes.c_uint8), ("scale_fmt", ctypes.c_uint8),
                ("reserved", ctypes.c_int8 * 4), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p)]


class RazerError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {razer_status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded librazer.so.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "python nvfp4_razer_w4a16_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
        P = ctypes.POINTER(razer_packed)
        for name in ("razer_quantize_weight", "razer_quantize_act"):
            f = getattr(L, name)
            f.restype, f.argtypes = i32, [vp, i32, P, vp, sz, vp]
        L.razer_quantize_act_noalloc.restype = i32
        L.razer_quantize_act_noalloc.argtypes = [vp, i32, P, vp]
        L.razer_dequant.restype, L.razer_dequant.argtypes = i32, [P, vp, i32, vp]
        L.razer_gemv.restype, L.razer_gemv.argtypes = i32, [vp, i32, P, vp, i32, vp, sz, vp]
        L.razer_gemv_group.restype = i32
        L.razer_gemv_group.argtypes = [vp, i32, ctypes.POINTER(P), ctypes.POINTER(vp), i32, i32, vp]
        L.razer_gemm.restype, L.razer_gemm.argtypes = i32, [vp, i32, i64, P, vp, i32, vp, sz, vp]
        L.razer_gemm_w4a4.restype, L.razer_gemm_w4a4.argtypes = i32, [P, P, vp, i32, vp, sz, vp]
        L.razer_weight_offset_sse.restype = i32
        L.razer_weight_offset_sse.argtypes = [vp, i32, i64, i64, i32, vp, vp, sz, vp]
        L.razer_workspace_bytes.restype = sz
        L.razer_workspace_bytes.argtypes = [i32, i64, i64, i64]
        L.razer_status_string.restype, L.razer_status_string.argtypes = ctypes.c_char_p, [i32]
        _lib = L
    return _lib


def razer_status_string(status: int) -> str:
    return lib().razer_status_string(int(status)).decode()


def razer_workspace_bytes(op: int, m: int, n: int, k: int) -> int:
    return int(lib().razer_workspace_bytes(op, m, n, k))


def _check(status: int, what: str):
    if status != RAZER_OK:
        raise RazerError(status, what)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}")
    return _DT[dt]


def _check_device(t: torch.Tensor, device: torch.device, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU, not {t.device}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, not {t.device}")


def _same_device(dev: torch.device, want: torch.device, name: str):
    if dev != want:
        raise ValueError(f"{name} must be on {want}, not {dev}")


def _check_buffer(t: torch.Tensor, shape, device: torch.device, name: str, dtype=None):
    """A caller-supplied output or workspace: the C ABI cannot see its size, so
    shape, dtype, device and contiguity are checked here, before any launch."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if dtype is None and shape is not None and t.dtype not in _DT:
        raise TypeError(f"{name}: unsupported dtype {t.dtype}")
    if device is not None:
        _check_device(t, device, name)


def _check_input(x: torch.Tensor, device: torch.device, name: str):
    _check_device(x, device, name)
    if x.dtype not in _DT:
        raise TypeError(f"{name}: unsupported dtype {x.dtype}")


class PackedTensor:
    """A RaZeR-packed tensor in device memory (torch tensors own the bytes).

    codes: uint8 [rows, cols // 2]; scales: uint8 [rows, cols // block] (two
    bytes per block, little-endian, for RAZER_SCALE_F16); tensor_scale: float32
    [1]; kind: RAZER_WEIGHT or RAZER_ACT; offsets: special-value offsets in
    units of 0.5; block: elements per block (16, 32, 64 or 128)."""

    def __init__(self, kind: int, rows: int, cols: int, offsets, device, flags: int = 0,
                 block: int = 16, scale_fmt: int = RAZER_SCALE_BYTE):
        if block not in BLOCK_SIZES:
            raise ValueError(f"block must be one of {BLOCK_SIZES}")
        if cols % block:
            raise ValueError("cols must be a multiple of the block size")
        self.kind, self.rows, self.cols, self.flags = kind, rows, cols, flags
        self.block, self.scale_fmt = block, scale_fmt
        self.offsets = tuple(int(o) for o in offsets)
        sbytes = 2 if scale_fmt == RAZER_SCALE_F16 else 1
        self.codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        self.scales = torch.empty((rows, cols // block * sbytes), dtype=torch.uint8, device=device)
        self.tensor_scale = torch.empty(1, dtype=torch.float32, device=device)

    @property
    def shape(self):
        return (self.rows, self.cols)

    def struct(self) -> razer_packed:
        s = razer_packed()
        s.kind, s.flags, s.rows, s.cols = self.kind, self.flags, self.rows, self.cols
        off = list(self.offsets) + [self.offsets[0]] * (2 - len(self.offsets))
        s.sv_off_half[0], s.sv_off_half[1] = off[0], off[1]
        s.block_log2, s.scale_fmt = self.block.bit_length() - 1, self.scale_fmt
        s.codes, s.scales = self.codes.data_ptr(), self.scales.data_ptr()
        s.tensor_scale = self.tensor_scale.data_ptr()
        return s

    def nbytes(self) -> int:
        return self.codes.numel() + self.scales.numel() + 4

    @property
    def device(self) -> torch.device:
        return self.codes.device

    def with_flags(self, flags: int) -> "PackedTensor":
        """The same tensor (buffers shared) with other descriptor flags, e.g.
        RAZER_FLAG_UNTRIMMED_PLAN for the products."""
        q = PackedTensor.__new__(PackedTensor)
        q.__dict__.update(self.__dict__)
        q.flags = flags
        return q

    def check(self, name: str = "packed tensor"):
        """Its buffers still match its shape and layout (they are plain
        attributes a caller can replace)."""
        sbytes = 2 if self.scale_fmt == RAZER_SCALE_F16 else 1
        bufs = ((self.codes, (self.rows, self.cols // 2), "codes"),
                (self.scales, (self.rows, self.cols // self.block * sbytes), "scales"),
                (self.tensor_scale, (1,), "tensor_scale"))
        for t, shape, what in bufs:
            _check_buffer(t, shape, None, f"{name}.{what}",
                          torch.float32 if what == "tensor_scale" else torch.uint8)
        dev = self.codes.device
        for t, _, what in bufs:
            _check_device(t, dev, f"{name}.{what}")
        return dev


def _workspace(op, m, n, k, device, workspace):
    need = razer_workspace_bytes(op, m, n, k)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    else:
        _check_buffer(workspace, None, device, "workspace")
    return workspace, workspace.numel() * workspace.element_size()


def _encoder_flags(remap: bool, four_over_six: bool, rescale: bool = False) -> int:
    if four_over_six:
        return RAZER_FLAG_FOUR_OVER_SIX
    if not remap:
        return RAZER_FLAG_NO_REMAP
    return RAZER_FLAG_RESCALE_LARGE_SV if rescale else 0


def _quantize(fn, op, kind, x, offsets, flags, out, workspace, stream, block, scale_fmt):
    if x.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    _check_input(x, x.device, "x")
    x = x.contiguous()
    rows, cols = x.shape
    if out is None:
        out = PackedTensor(kind, rows, cols, offsets, x.device, flags, block, scale_fmt)
    elif (out.rows, out.cols) != (rows, cols):
        raise ValueError(f"out is {out.rows}x{out.cols}, the input {rows}x{cols}")
    else:
        _same_device(out.check("out"), x.device, "out")
    s = out.struct()
    ws, wsb = _workspace(op, rows, 0, cols, x.device, workspace)
    _check(fn(ctypes.c_void_p(x.data_ptr()), _dtype_code(x.dtype), ctypes.byref(s),
              ctypes.c_void_p(ws.data_ptr() if ws is not None else 0), wsb,
              ctypes.c_void_p(_stream(stream))), fn.__name__)
    return out


def razer_quantize_weight(w: torch.Tensor, offsets=DEFAULT_WEIGHT_OFFSETS, remap: bool = True,
                          out: PackedTensor | None = None, workspace=None, stream=None,
                          four_over_six: bool = False, block: int = 16,
                          scale_fmt: int = RAZER_SCALE_BYTE, rescale: bool = False):
    """Offline RaZeR weight encoding of w [N, K] (fp32/fp16/bf16, on the GPU).
    remap=False gives plain NVFP4, four_over_six=True the Four Over Six
    baseline, rescale=True RaZeR with rescaled large special values (a
    candidate with |v| > 6 maps the block maximum to |v|; 16-element blocks,
    byte scales); block / scale_fmt pick a layout variant; a given `out`
    carries its own flags and layout instead."""
    return _quantize(lib().razer_quantize_weight, RAZER_OP_QUANTIZE_WEIGHT, RAZER_WEIGHT, w,
                     offsets, _encoder_flags(remap, four_over_six, rescale), out, workspace, stream,
                     block, scale_fmt)


def razer_quantize_act(x: torch.Tensor, offsets=DEFAULT_ACT_OFFSETS, remap: bool = True,
                       out: PackedTensor | None = None, workspace=None, stream=None,
                       four_over_six: bool = False, block: int = 16, rescale: bool = False):
    """Online RaZeR activation encoding of x [rows, cols] (fp16/bf16, on the GPU).
    remap / four_over_six / rescale / block / out as for razer_quantize_weight."""
    return _quantize(lib().razer_quantize_act, RAZER_OP_QUANTIZE_ACT, RAZER_ACT, x, offsets,
                     _encoder_flags(remap, four_over_six, rescale), out, workspace, stream, block,
                     RAZER_SCALE_BYTE)


def razer_quantize_act_noalloc(x: torch.Tensor, out: PackedTensor, stream=None):
    """razer_quantize_act into a caller-allocated `out` without a workspace
    (the library's per-device static scratch holds the partials): for code
    that cannot allocate, e.g. under graph capture.  Calls that overlap on one
    device race on that scratch."""
    if x.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    _check_input(x, x.device, "x")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (a copy would allocate)")
    if (out.rows, out.cols) != tuple(x.shape):
        raise ValueError(f"out is {out.rows}x{out.cols}, the input {tuple(x.shape)}")
    _same_device(out.check("out"), x.device, "out")
    s = out.struct()
    _check(lib().razer_quantize_act_noalloc(ctypes.c_void_p(x.data_ptr()), _dtype_code(x.dtype),
                                            ctypes.byref(s), ctypes.c_void_p(_stream(stream))),
           "razer_quantize_act_noalloc")
    return out


def razer_dequant(t: PackedTensor, dtype: torch.dtype = torch.float32, out=None, stream=None):
    dev = t.check("t")
    if out is None:
        out = torch.empty((t.rows, t.cols), dtype=dtype, device=dev)
    else:
        _check_buffer(out, (t.rows, t.cols), dev, "out")
    s = t.struct()
    _check(lib().razer_dequant(ctypes.byref(s), ctypes.c_void_p(out.data_ptr()),
                               _dtype_code(out.dtype), ctypes.c_void_p(_stream(stream))),
           "razer_dequant")
    return out


def razer_gemv(x: torch.Tensor, w: PackedTensor, out_dtype: torch.dtype | None = None, out=None,
               workspace=None, stream=None):
    """y[N] = x[K] . W^T for a packed weight W [N, K]."""
    dev = w.check("w")
    _check_input(x, dev, "x")
    x = x.contiguous()
    if x.numel() != w.cols:
        raise ValueError("x must hold K elements")
    if out is None:
        out = torch.empty(w.rows, dtype=out_dtype or x.dtype, device=x.device)
    else:
        _check_buffer(out, None, dev, "out")
        if out.numel() != w.rows or out.dtype not in _DT:
            raise ValueError(f"out must hold N = {w.rows} elements of f32, f16 or bf16")
    ws, wsb = _workspace(RAZER_OP_GEMV, 1, w.rows, w.cols, x.device, workspace)
    s = w.struct()
    _check(lib().razer_gemv(ctypes.c_void_p(x.data_ptr()), _dtype_code(x.dtype), ctypes.byref(s),
                            ctypes.c_void_p(out.data_ptr()), _dtype_code(out.dtype),
                            ctypes.c_void_p(ws.data_ptr() if ws is not None else 0), wsb,
                            ctypes.c_void_p(_stream(stream))), "razer_gemv")
    return out


RAZER_GEMV_GROUP_MAX = 4


def razer_gemv_group(x: torch.Tensor, ws, out_dtype: torch.dtype | None = None, outs=None,
                     stream=None):
    """[x[K] . W^T for W in ws] in one launch (weights sharing x, e.g. gate and up)."""
    ws = list(ws)
    if not 1 <= len(ws) <= RAZER_GEMV_GROUP_MAX:
        raise ValueError(f"1..{RAZER_GEMV_GROUP_MAX} weights")
    dev = ws[0].check("ws[0]")
    for i, w in enumerate(ws):
        _same_device(w.check(f"ws[{i}]"), dev, f"ws[{i}]")
    _check_input(x, dev, "x")
    x = x.contiguous()
    if any(w.cols != x.numel() for w in ws):
        raise ValueError("x must hold K elements for every weight")
    if outs is None:
        outs = [torch.empty(w.rows, dtype=out_dtype or x.dtype, device=x.device) for w in ws]
    else:
        outs = list(outs)
        if len(outs) != len(ws):
            raise ValueError("one output per weight")
        for i, (o, w) in enumerate(zip(outs, ws)):
            _check_buffer(o, None, dev, f"outs[{i}]")
            if o.numel() != w.rows:
                raise ValueError(f"outs[{i}] must hold {w.rows} elements")
            if o.dtype != outs[0].dtype or o.dtype not in _DT:
                raise ValueError("every output must have the same dtype (f32, f16 or bf16)")
    structs = [w.struct() for w in ws]
    ptrs = (ctypes.POINTER(razer_packed) * len(ws))(*[ctypes.pointer(s) for s in structs])
    ys = (ctypes.c_void_p * len(ws))(*[o.data_ptr() for o in outs])
    _check(lib().razer_gemv_group(ctypes.c_void_p(x.data_ptr()), _dtype_code(x.dtype), ptrs, ys,
                                  len(ws), _dtype_code(outs[0].dtype), ctypes.c_void_p(_stream(stream))),
           "razer_gemv_group")
    return outs


def razer_gemm(x: torch.Tensor, w: PackedTensor, out_dtype: torch.dtype | None = None, out=None,
               workspace=None, stream=None):
    """y[M, N] = x[M, K] . W^T for a packed weight W [N, K]."""
    dev = w.check("w")
    _check_input(x, dev, "x")
    x = x.contiguous()
    if x.dim() != 2 or x.shape[1] != w.cols:
        raise ValueError("x must be [M, K]")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, w.rows), dtype=out_dtype or x.dtype, device=x.device)
    else:
        _check_buffer(out, (m, w.rows), dev, "out")
    op = RAZER_OP_GEMM_UNTRIMMED if w.flags & RAZER_FLAG_UNTRIMMED_PLAN else RAZER_OP_GEMM
    ws, wsb = _workspace(op, m, w.rows, w.cols, x.device, workspace)
    s = w.struct()
    _check(lib().razer_gemm(ctypes.c_void_p(x.data_ptr()), _dtype_code(x.dtype), m, ctypes.byref(s),
                            ctypes.c_void_p(out.data_ptr()), _dtype_code(out.dtype),
                            ctypes.c_void_p(ws.data_ptr() if ws is not None else 0), wsb,
                            ctypes.c_void_p(_stream(stream))), "razer_gemm")
    return out


def razer_weight_offset_sse(w: torch.Tensor, off0: int = DEFAULT_WEIGHT_OFFSETS[0], out=None,
                            workspace=None, stream=None) -> torch.Tensor:
    """Total squared reconstruction error of w [N, K] encoded with offsets
    (off0, o), for o = -7..7 (device float64 [15], entry o + 7)."""
    if w.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    _check_input(w, w.device, "w")
    w = w.contiguous()
    rows, cols = w.shape
    if out is None:
        out = torch.empty(len(SECOND_PAIR_OFFSETS), dtype=torch.float64, device=w.device)
    else:
        _check_buffer(out, (len(SECOND_PAIR_OFFSETS),), w.device, "out", torch.float64)
    ws, wsb = _workspace(RAZER_OP_OFFSET_SEARCH, 0, rows, cols, w.device, workspace)
    _check(lib().razer_weight_offset_sse(ctypes.c_void_p(w.data_ptr()), _dtype_code(w.dtype), rows, cols,
                                         int(off0), ctypes.c_void_p(out.data_ptr()),
                                         ctypes.c_void_p(ws.data_ptr() if ws is not None else 0), wsb,
                                         ctypes.c_void_p(_stream(stream))), "razer_weight_offset_sse")
    return out


def razer_best_second_offset(w: torch.Tensor, off0: int = DEFAULT_WEIGHT_OFFSETS[0], stream=None):
    """(offset with the lowest total error -- ties to the lowest offset, the 15
    errors on the host).  Waits for the result."""
    sse = razer_weight_offset_sse(w, off0, stream=stream).cpu()
    return SECOND_PAIR_OFFSETS[int(torch.argmin(sse))], sse


def razer_gemm_w4a4(x: PackedTensor, w: PackedTensor, out_dtype: torch.dtype = torch.bfloat16, out=None,
                    workspace=None, stream=None):
    """y[M, N] = dequant(x)[M, K] . dequant(w)^T for packed x [M, K] (normally an
    activation encoding) and packed w [N, K]."""
    if x.cols != w.cols:
        raise ValueError("x and w must have the same K")
    dev = x.check("x")
    _same_device(w.check("w"), dev, "w")
    if out is None:
        out = torch.empty((x.rows, w.rows), dtype=out_dtype, device=dev)
    else:
        _check_buffer(out, (x.rows, w.rows), dev, "out")
    need = razer_workspace_bytes(RAZER_OP_GEMM_W4A4, x.rows, w.rows, w.cols)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace is not None:
        _check_buffer(workspace, None, dev, "workspace")
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    sx, sw = x.struct(), w.struct()
    _check(lib().razer_gemm_w4a4(ctypes.byref(sx), ctypes.byref(sw), ctypes.c_void_p(out.data_ptr()),
                                 _dtype_code(out.dtype),
                                 ctypes.c_void_p(workspace.data_ptr() if workspace is not None else 0), wsb,
                                 ctypes.c_void_p(_stream(stream))), "razer_gemm_w4a4")
    return out
