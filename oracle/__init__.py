"""CPU oracle for RaZeR-NVFP4 -- test infrastructure only.

A ctypes wrapper around ``razer_oracle.c``: a plain single-threaded C statement
of the RaZeR-NVFP4 encoder, decoder and W4A16 product, written from the pages
("RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
Remapping", papernotes.org notes; and the gist.science technical summary of the
same paper).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
never imports, links or calls it, and the two share no code.

All arrays are numpy host arrays.  fp16/bf16 inputs are widened to fp32 by the
caller (exact).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "razer_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

WEIGHT = 0
ACT = 1
SCALE_BYTE, SCALE_F16 = 0, 1  # block-scale storage: one E3M3/E4M3 byte, or the FP16 group scale
BLOCK_SIZES = (16, 32, 64, 128)


def build_oracle() -> str:
    """Compile the oracle with gcc: -O2, no fast-math, no FP contraction."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """Load liboracle.so, building it first only if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_oracle()
        L = ctypes.CDLL(_LIB)
        d, i, i64, f = ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        vp = ctypes.c_void_p
        L.rzo_fp4_value.restype = d
        L.rzo_fp4_value.argtypes = [i]
        L.rzo_fp4_round_mag.restype = i
        L.rzo_fp4_round_mag.argtypes = [d]
        L.rzo_scale_value.restype = d
        L.rzo_scale_value.argtypes = [i, i]
        L.rzo_scale_round.restype = i
        L.rzo_scale_round.argtypes = [i, f]
        L.rzo_scale_max.restype = d
        L.rzo_scale_max.argtypes = [i]
        L.rzo_special_value.restype = d
        L.rzo_special_value.argtypes = [i, i]
        L.rzo_encode_block_scaled.restype = None
        L.rzo_encode_block_scaled.argtypes = [vp, i, vp, i, i, vp, vp]
        L.rzo_quantize.restype = i
        L.rzo_quantize.argtypes = [i, vp, i64, i64, vp, i, vp, vp, vp]
        L.rzo_decode_value.restype = d
        L.rzo_decode_value.argtypes = [i, i, i, vp]
        L.rzo_block_scale.restype = d
        L.rzo_block_scale.argtypes = [i, i]
        L.rzo_dequant_f64.restype = None
        L.rzo_dequant_f64.argtypes = [i, vp, vp, f, vp, i64, i64, vp]
        L.rzo_dequant_f32.restype = None
        L.rzo_dequant_f32.argtypes = [i, vp, vp, f, vp, i64, i64, vp]
        L.rzo_scale_value_fmt.restype = d
        L.rzo_scale_value_fmt.argtypes = [i, i, i]
        L.rzo_scale_round_fmt.restype = i
        L.rzo_scale_round_fmt.argtypes = [i, i, f]
        L.rzo_scale_max_fmt.restype = d
        L.rzo_scale_max_fmt.argtypes = [i, i]
        L.rzo_quantize_fmt.restype = i
        L.rzo_quantize_fmt.argtypes = [i, vp, i64, i64, vp, i, i, i, vp, vp, vp]
        for name in ("rzo_dequant_fmt_f64", "rzo_dequant_fmt_f32"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [i, i, i, vp, vp, f, vp, i64, i64, vp]
        L.rzo_gemm.restype = None
        L.rzo_gemm.argtypes = [vp, i64, i64, i, vp, vp, f, vp, i64, vp, i64, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _offsets(kind: int, offsets) -> np.ndarray:
    off = np.zeros(2, dtype=np.int8)
    vals = list(offsets)
    if kind == WEIGHT and len(vals) != 2:
        raise ValueError("weights take two offsets")
    if kind == ACT and len(vals) != 1:
        raise ValueError("activations take one offset")
    off[: len(vals)] = vals
    return off


# ---- scalar helpers ---------------------------------------------------------

def fp4_value(code: int) -> float:
    return lib().rzo_fp4_value(code)


def fp4_round_mag(a: float) -> int:
    return lib().rzo_fp4_round_mag(float(a))


def scale_value(kind: int, code: int) -> float:
    return lib().rzo_scale_value(kind, code)


def scale_round(kind: int, v: float) -> int:
    return lib().rzo_scale_round(kind, float(np.float32(v)))


def scale_max(kind: int) -> float:
    return lib().rzo_scale_max(kind)


def scale_value_fmt(kind: int, sfmt: int, code: int) -> float:
    return lib().rzo_scale_value_fmt(kind, sfmt, code)


def scale_round_fmt(kind: int, sfmt: int, v: float) -> int:
    return lib().rzo_scale_round_fmt(kind, sfmt, float(np.float32(v)))


def scale_max_fmt(kind: int, sfmt: int) -> float:
    return lib().rzo_scale_max_fmt(kind, sfmt)


def special_value(neg: int, off_half: int) -> float:
    return lib().rzo_special_value(neg, off_half)


def decode_value(kind: int, code: int, sbyte: int, offsets) -> float:
    off = _offsets(kind, offsets)
    return lib().rzo_decode_value(kind, code, sbyte, _ptr(off))


def block_scale(kind: int, sbyte: int) -> float:
    return lib().rzo_block_scale(kind, sbyte)


# ---- block and tensor entry points -------------------------------------------

def encode_block_scaled(y, candidates, remap: bool = True):
    """Remap one block of already-scaled values; returns (codes[n], sel)."""
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    cand = np.ascontiguousarray(np.asarray(candidates, dtype=np.float64))
    if y.size > 128:
        raise ValueError("at most 128 values per block")
    codes = np.zeros(y.size, dtype=np.uint8)
    sel = ctypes.c_int(0)
    lib().rzo_encode_block_scaled(_ptr(y), y.size, _ptr(cand), cand.size, int(remap), _ptr(codes),
                                  ctypes.byref(sel))
    return codes, sel.value


class Packed:
    """Host copy of a packed RaZeR tensor."""

    def __init__(self, kind, rows, cols, offsets, codes, scales, tensor_scale, block=16,
                 scale_fmt=SCALE_BYTE):
        self.kind, self.rows, self.cols = kind, rows, cols
        self.offsets = tuple(int(o) for o in offsets)
        self.codes, self.scales = codes, scales  # scales: uint8, or uint16 for SCALE_F16
        self.tensor_scale = np.float32(tensor_scale)
        self.block, self.scale_fmt = block, scale_fmt

    def unpacked_codes(self) -> np.ndarray:
        c = self.codes.reshape(self.rows, self.cols // 2)
        out = np.empty((self.rows, self.cols), dtype=np.uint8)
        out[:, 0::2] = c & 15
        out[:, 1::2] = c >> 4
        return out


MODE_PLAIN, MODE_RAZER, MODE_FOUR_OVER_SIX, MODE_RAZER_RESCALE = 0, 1, 2, 3


def quantize(kind: int, x, offsets, remap: bool = True, four_over_six: bool = False,
             block: int = 16, scale_fmt: int = SCALE_BYTE, rescale: bool = False) -> Packed:
    """Encode x (RaZeR, plain NVFP4 when not remap, or the Four Over Six
    baseline when four_over_six: plain FP4 with a per-block choice of the
    max -> 6 or max -> 4 scale), with `block` elements per block and byte or
    FP16 group scales.  rescale (RaZeR, 16-element blocks, byte scales): every
    candidate is tried on its own, one with |v| > 6 at the block scale that maps
    the block maximum to |v|, and the encoding with the smallest squared error
    in real units is kept."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    off = _offsets(kind, offsets)
    codes = np.zeros(rows * cols // 2, dtype=np.uint8)
    nblk = rows * cols // block if block in BLOCK_SIZES else 0
    scales = np.zeros(nblk, dtype=np.uint16 if scale_fmt == SCALE_F16 else np.uint8)
    ts = np.zeros(1, dtype=np.float32)
    mode = (MODE_FOUR_OVER_SIX if four_over_six else
            (MODE_PLAIN if not remap else MODE_RAZER_RESCALE if rescale else MODE_RAZER))
    rc = lib().rzo_quantize_fmt(kind, _ptr(x), rows, cols, _ptr(off), mode, block, scale_fmt,
                                _ptr(codes), _ptr(scales), _ptr(ts))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return Packed(kind, rows, cols, offsets, codes, scales, ts[0], block, scale_fmt)


def quantize_weight(w, offsets=(-2, 4), remap: bool = True, four_over_six: bool = False,
                    rescale: bool = False) -> Packed:
    return quantize(WEIGHT, w, offsets, remap, four_over_six, rescale=rescale)


def quantize_act(x, offsets=(-2,), remap: bool = True, four_over_six: bool = False,
                 rescale: bool = False) -> Packed:
    return quantize(ACT, x, offsets, remap, four_over_six, rescale=rescale)


SECOND_PAIR_OFFSETS = tuple(range(-7, 8))  # offsets tried for the second weight pair


def weight_offset_sse(w, off0: int = -2) -> np.ndarray:
    """Total squared reconstruction error of a weight tensor for every
    second-pair offset.

    "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
    Remapping" (papernotes.org notes), Loss function / training strategy: the
    extra weight pair is chosen offline by a grid search (one pair per model,
    e.g. +/-5 with +/-8 for Llama).  Data-free reading: for each offset o in
    -7..7 the tensor is encoded with offsets (off0, o) and dequantized in fp64;
    entry o + 7 is sum((w - dequant)^2) in fp64.  A non-finite tensor gives NaN
    everywhere."""
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float32))
    w64 = w.astype(np.float64)
    out = np.empty(len(SECOND_PAIR_OFFSETS), dtype=np.float64)
    for i, o in enumerate(SECOND_PAIR_OFFSETS):
        d = dequant_f64(quantize_weight(w, (off0, o)))
        out[i] = np.sum((w64 - d) ** 2)
    return out


def best_second_offset(w, off0: int = -2):
    """(offset with the lowest total error, the 15 errors); ties go to the
    lowest offset."""
    sse = weight_offset_sse(w, off0)
    return SECOND_PAIR_OFFSETS[int(np.argmin(sse))], sse


def dequant_f64(p: Packed) -> np.ndarray:
    out = np.empty((p.rows, p.cols), dtype=np.float64)
    off = _offsets(p.kind, p.offsets)
    lib().rzo_dequant_fmt_f64(p.kind, p.block, p.scale_fmt, _ptr(p.codes), _ptr(p.scales),
                              float(p.tensor_scale), _ptr(off), p.rows, p.cols, _ptr(out))
    return out


def dequant_f32(p: Packed) -> np.ndarray:
    out = np.empty((p.rows, p.cols), dtype=np.float32)
    off = _offsets(p.kind, p.offsets)
    lib().rzo_dequant_fmt_f32(p.kind, p.block, p.scale_fmt, _ptr(p.codes), _ptr(p.scales),
                              float(p.tensor_scale), _ptr(off), p.rows, p.cols, _ptr(out))
    return out


def _default_layout(p: Packed):
    if p.block != 16 or p.scale_fmt != SCALE_BYTE:
        raise ValueError("the products take 16-element blocks with byte scales")


def gemm(x, p: Packed, cols=None):
    """fp64 product y = x @ w^T over the packed weight, plus the norm sum |x||w|.

    ``cols`` selects weight rows (output columns); None means all.  Returns
    (y [m, ncols], norm [m, ncols])."""
    _default_layout(p)
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    if k != p.cols:
        raise ValueError("inner dimensions differ")
    off = _offsets(p.kind, p.offsets)
    if cols is None:
        idx = None
        ncols = p.rows
    else:
        idx = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
        ncols = idx.size
    y = np.zeros((m, ncols), dtype=np.float64)
    nrm = np.zeros((m, ncols), dtype=np.float64)
    lib().rzo_gemm(_ptr(x), m, k, p.kind, _ptr(p.codes), _ptr(p.scales), float(p.tensor_scale),
                   _ptr(off), p.rows, None if idx is None else _ptr(idx), ncols, _ptr(y), _ptr(nrm))
    return y, nrm


def gemm_pairs(x, p: Packed, rows_m, cols_n):
    """The product oracle at individual outputs: y[i] = x[rows_m[i]] . w[cols_n[i]]
    and its norm, for sampled (m, n) pairs of a large product.  Returns
    (y [npairs], norm [npairs])."""
    _default_layout(p)
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if x.ndim != 2 or x.shape[1] != p.cols:
        raise ValueError("x must be [m, K]")
    rows_m = np.asarray(rows_m, dtype=np.int64)
    cols_n = np.asarray(cols_n, dtype=np.int64)
    off = _offsets(p.kind, p.offsets)
    y = np.zeros(rows_m.size, dtype=np.float64)
    nrm = np.zeros(rows_m.size, dtype=np.float64)
    one_y, one_n = np.zeros(1, np.float64), np.zeros(1, np.float64)
    for i, (mi, ni) in enumerate(zip(rows_m, cols_n)):
        xr = np.ascontiguousarray(x[mi])
        idx = np.array([ni], dtype=np.int64)
        lib().rzo_gemm(_ptr(xr), 1, p.cols, p.kind, _ptr(p.codes), _ptr(p.scales), float(p.tensor_scale),
                       _ptr(off), p.rows, _ptr(idx), 1, _ptr(one_y), _ptr(one_n))
        y[i], nrm[i] = one_y[0], one_n[0]
    return y, nrm


def gemm_any(x, p: Packed, cols=None):
    """fp64 product y = x @ w^T and norm |x| @ |w|^T over the exactly decoded
    weights of any layout (block sizes, FP16 group scales): the oracle's
    decoder followed by a numpy matmul.  ``cols`` selects weight rows (output
    columns); None means all.  Returns (y [m, ncols], norm [m, ncols])."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    w = dequant_f64(p if cols is None else select_rows(p, cols))
    return x @ w.T, np.abs(x) @ np.abs(w).T


def gemm_w4a4(xp: Packed, wp: Packed, cols=None):
    """fp64 product of two packed tensors, y = dequant(x) @ dequant(w)^T, plus
    the norm sum |dequant(x)| |dequant(w)|.

    "RaZeR: Pushing the Limits of NVFP4 Quantization with Redundant Zero
    Remapping" (papernotes.org notes), Overall framework and Key designs 1-2:
    in W4A4 the activations carry the online 2-candidate encoding and the
    weights the offline 4-candidate one; the product is over the decoded
    values.  ``cols`` selects weight rows (output columns).  Returns
    (y [m, ncols], norm [m, ncols])."""
    _default_layout(xp)
    _default_layout(wp)
    if xp.cols != wp.cols:
        raise ValueError("inner dimensions differ")
    xd = dequant_f64(xp)
    if cols is not None:  # decode only the selected weight rows (same tensor scale)
        wp = select_rows(wp, cols)
    wd = dequant_f64(wp)
    return xd @ wd.T, np.abs(xd) @ np.abs(wd).T


def select_rows(p: Packed, idx) -> Packed:
    """The packed rows idx of a tensor of any layout (same tensor scale,
    offsets and layout), for decoding a sample of a large tensor."""
    idx = np.asarray(idx, dtype=np.int64)
    return Packed(p.kind, idx.size, p.cols, p.offsets,
                  np.ascontiguousarray(p.codes.reshape(p.rows, p.cols // 2)[idx]).reshape(-1),
                  np.ascontiguousarray(p.scales.reshape(p.rows, p.cols // p.block)[idx]).reshape(-1),
                  p.tensor_scale, p.block, p.scale_fmt)


def gemm_w4a4_pairs(xp: Packed, wp: Packed, rows_m, cols_n):
    """gemm_w4a4 at individual outputs (m, n): the decoded rows' fp64 dot
    products and norms.  Returns (y [npairs], norm [npairs])."""
    if xp.cols != wp.cols:
        raise ValueError("inner dimensions differ")
    xd = dequant_f64(select_rows(xp, rows_m))
    wd = dequant_f64(select_rows(wp, cols_n))
    return np.einsum("ik,ik->i", xd, wd), np.einsum("ik,ik->i", np.abs(xd), np.abs(wd))
