"""Seeded synthetic inputs shaped like the LLM tensors RaZeR is evaluated on.

This module holds random-number generation only (no quantization arithmetic),
so that the GPU library and the CPU oracle can be fed the very same tensors.
Every tensor comes from a counter-based Philox stream with seed
``1000 * config_id + tensor_id`` and is generated in fixed-size chunks, so the
values do not depend on the caller.  Weights come back as fp32 (they are
quantized by the weight encoder); activations are rounded to fp16/bf16 with
round-to-nearest-even.

Workloads (stand-ins for the model weights and activations of the paper's
Llama-3 / Qwen-3 experiments, which are not available here):

==  =====================  ==========================================================
id  name                   tensors
==  =====================  ==========================================================
0   pr1_tiny               W[256,1024] ~ N(0, 0.02), 0.1% entries x10; x[1,1024] fp16 N(0,1)
1   llama3_8b_decode       x[1,K] fp16 N(0,1), 8 channels x20; W = 0.02 * t(5):
                           gate/up [14336,4096], down [4096,14336], qkv [6144,4096]
2   small_batch            x bf16 [M,K] N(0,1) (first M rows of a [32,K] draw);
                           W ~ N(0, 0.015), 0.05% entries x15: [4096,4096], [28672,8192]
3   act_quant              X bf16 [4096, 8192] N(0,1); 16 channels x50; 1% tokens x5
4   prefill                x bf16 [2048, 8192] N(0,1); W = 0.015 * t(4) fp32 [28672, 8192]
==  =====================  ==========================================================
"""
from __future__ import annotations

import numpy as np
import torch

CHUNK = 1 << 22  # elements per generation chunk

CONFIG_IDS = {"pr1_tiny": 0, "llama3_8b_decode": 1, "small_batch": 2, "act_quant": 3, "prefill": 4}

# Tensor ids within a configuration.
T_W, T_X, T_W_OUTLIER, T_X_CHANNELS, T_X_TOKENS = 0, 1, 2, 3, 4


def seed_for(config: str | int, tensor_id: int, sub: int = 0) -> int:
    cid = CONFIG_IDS[config] if isinstance(config, str) else int(config)
    return 1000 * cid + tensor_id + 100 * sub


def _gen(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(seed))


def _normal(n: int, seed: int) -> np.ndarray:
    g = _gen(seed)
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        out[s:e] = g.standard_normal(e - s, dtype=np.float32)
    return out


def _student_t(n: int, nu: float, seed: int) -> np.ndarray:
    g = _gen(seed)
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        out[s:e] = g.standard_t(nu, size=e - s).astype(np.float32)
    return out


def _distinct(n: int, count: int, seed: int) -> np.ndarray:
    """`count` distinct indices in [0, n), seeded."""
    if count <= 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_gen(seed).choice(n, size=count, replace=False)).astype(np.int64)


def weight_normal(rows: int, cols: int, std: float, outlier_frac: float, outlier_mult: float,
                  seed: int, seed_outlier: int) -> np.ndarray:
    w = _normal(rows * cols, seed)
    w *= np.float32(std)
    cnt = int(round(outlier_frac * rows * cols))
    idx = _distinct(rows * cols, cnt, seed_outlier)
    w[idx] *= np.float32(outlier_mult)
    return w.reshape(rows, cols)


def weight_student_t(rows: int, cols: int, nu: float, scale: float, seed: int) -> np.ndarray:
    w = _student_t(rows * cols, nu, seed)
    w *= np.float32(scale)
    return w.reshape(rows, cols)


def activations(rows: int, cols: int, seed: int, dtype: torch.dtype, channels: int = 0,
                channel_mult: float = 1.0, seed_channels: int = 0, tokens: int = 0,
                token_mult: float = 1.0, seed_tokens: int = 0) -> torch.Tensor:
    x = _normal(rows * cols, seed).reshape(rows, cols)
    if channels:
        ch = _distinct(cols, channels, seed_channels)
        x[:, ch] *= np.float32(channel_mult)
    if tokens:
        tk = _distinct(rows, tokens, seed_tokens)
        x[tk, :] *= np.float32(token_mult)
    return torch.from_numpy(x).to(dtype)  # round to nearest even


# ---- the five workloads ---------------------------------------------------------

def pr1_tiny():
    """Tiny weight W[256,1024] and fp16 x[1,1024]."""
    w = weight_normal(256, 1024, 0.02, 0.001, 10.0, seed_for(0, T_W), seed_for(0, T_W_OUTLIER))
    x = activations(1, 1024, seed_for(0, T_X), torch.float16)
    return w, x


LLAMA3_8B_DECODE = {"qkv": (6144, 4096), "gate": (14336, 4096), "up": (14336, 4096),
                    "down": (4096, 14336)}


def llama3_8b_decode_weight(name: str) -> np.ndarray:
    n, k = LLAMA3_8B_DECODE[name]
    sub = list(LLAMA3_8B_DECODE).index(name)
    return weight_student_t(n, k, 5.0, 0.02, seed_for(1, T_W, sub))


def llama3_8b_decode_x(k: int) -> torch.Tensor:
    sub = 0 if k == 4096 else 1
    return activations(1, k, seed_for(1, T_X, sub), torch.float16, channels=8, channel_mult=20.0,
                       seed_channels=seed_for(1, T_X_CHANNELS, sub))


SMALL_BATCH_SHAPES = ((4096, 4096), (28672, 8192))
SMALL_BATCH_M = (1, 2, 4, 8, 16, 32)


def small_batch_weight(n: int, k: int) -> np.ndarray:
    sub = SMALL_BATCH_SHAPES.index((n, k))
    return weight_normal(n, k, 0.015, 0.0005, 15.0, seed_for(2, T_W, sub),
                         seed_for(2, T_W_OUTLIER, sub))


def small_batch_x(m: int, k: int) -> torch.Tensor:
    sub = 0 if k == 4096 else 1
    return activations(32, k, seed_for(2, T_X, sub), torch.bfloat16)[:m].contiguous()


def act_quant_x(tokens: int = 4096, hidden: int = 8192) -> torch.Tensor:
    return activations(tokens, hidden, seed_for(3, T_X), torch.bfloat16, channels=16,
                       channel_mult=50.0, seed_channels=seed_for(3, T_X_CHANNELS),
                       tokens=int(round(0.01 * tokens)), token_mult=5.0,
                       seed_tokens=seed_for(3, T_X_TOKENS))


def prefill_weight(n: int = 28672, k: int = 8192) -> np.ndarray:
    return weight_student_t(n, k, 4.0, 0.015, seed_for(4, T_W))


def prefill_x(m: int = 2048, k: int = 8192) -> torch.Tensor:
    return activations(m, k, seed_for(4, T_X), torch.bfloat16)


def checksum(a) -> str:
    """Short content hash of a tensor/array, for logging which inputs were used."""
    import hashlib
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().contiguous().view(torch.uint8).numpy()
    return hashlib.sha1(np.ascontiguousarray(a).view(np.uint8).tobytes()).hexdigest()[:12]
