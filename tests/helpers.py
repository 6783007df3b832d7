"""Shared test helpers: raw-bit views, host pools, and the scenario runner that drives either block
manager (the oracle's model or the product's C++ one) through the same sequence of operations."""
from __future__ import annotations

import numpy as np
import torch

RAW_NP = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


def raw(t: torch.Tensor) -> np.ndarray:
    """numpy view of a CPU tensor's raw elements (float32 values, or uint16 bits of f16/bf16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(t.dtype)


def host_pool(num_blocks: int, H: int, D: int, dtype: str, B: int = 16, fill=None) -> np.ndarray:
    n = num_blocks * H * B * D
    a = np.zeros(n, RAW_NP[dtype])
    if fill is not None:
        a[:] = fill
    return a


def nan_bits(dtype: str):
    return {"f32": np.float32(np.nan), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0),
            "fp8": np.uint8(0x7F)}[dtype]


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def max_abs_err(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2, "fp8": 3e-2}
