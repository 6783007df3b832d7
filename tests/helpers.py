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


def plan_order_model(lens, pt, H, base, prefix, round_items, max_len):
    """pa_decode_plan's dealing order written out: sequences by the 16-position steps of their
    largest partition, largest first (ties in batch order); with more than one and at most two
    rounds of round_items items, the largest on the one-item wavefronts, the next largest in the
    two-item wavefronts' first round and the rest smallest first; otherwise rounds filled
    alternately from the largest and the smallest left.  Partitions of pt positions after `base`
    (a shared prefix of that length when `prefix`), H items per partition."""
    items, steps = [], []
    for L in np.clip(lens, 0, max_len):
        L = int(L)
        n = -(-(L - base) // pt) if L > base else (0 if prefix else 1)
        items.append(n * H)
        steps.append(-(-(-(-(L - base) // 16)) // n) if L > base else 0)
    rest = sorted(range(len(lens)), key=lambda s: -steps[s])  # stable
    total = sum(items)
    if round_items < total <= 2 * round_items:
        # two rounds: the largest sequences on the one-item wavefronts, the next largest in the
        # two-item wavefronts' first round, the rest smallest first
        pairs, singles = total - round_items, 2 * round_items - total
        first, single, second, nf, ns = [], [], [], 0, 0
        for s in rest:
            if ns + items[s] <= singles:
                single.append(s)
                ns += items[s]
            elif nf + items[s] <= pairs:
                first.append(s)
                nf += items[s]
            else:
                second.append(s)
        return first + single + second[::-1]
    out, rnd = [], 0
    while rest:
        n = 0
        while rest and n < round_items:
            s = rest.pop(0) if rnd % 2 == 0 else rest.pop()
            out.append(s)
            n += items[s]
        rnd += 1
    return out
