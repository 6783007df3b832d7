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


def plan_busiest_steps(lens, pt, H, order, round_items, max_len):
    """16-position steps of the busiest wavefront when the items of `order` (each sequence's
    partitions times H, every one at its largest partition's steps) are dealt item f -> wavefront
    f mod round_items, one by one."""
    load = np.zeros(round_items, np.int64)
    f = 0
    for s in order:
        L = int(min(max(int(lens[s]), 0), max_len))
        n = -(-L // pt) if L > 0 else 1
        steps = -(-(-(-L // 16)) // n) if L > 0 else 0
        for _ in range(n * H):
            load[f % round_items] += steps
            f += 1
    return int(load.max())


def plan_partition_model(lens, auto, H, round_items, step_bytes, max_len, round_bytes=240 * 1024):
    """pa_decode_plan's partition size for an automatic call without a prefix: the sizes auto,
    auto + 64, ... up to 2,048 while the list keeps more than one round, each costed as the busiest
    wavefront's KV bytes under the planned deal plus round_bytes per round of items; the cheapest
    (the first of equals), or 0 where that is auto itself."""
    best, pick = None, auto
    for c in range(auto, max(auto, 2048) + 1, 64):
        total = sum((-(-int(min(max(L, 0), max_len)) // c) if L > 0 else 1) * H for L in lens)
        if total <= round_items:
            break
        order = plan_order_model(lens, c, H, 0, False, round_items, max_len)
        cost = plan_busiest_steps(lens, c, H, order, round_items, max_len) * step_bytes + \
            round_bytes * total / round_items
        if best is None or cost < best:
            best, pick = cost, c
    return 0 if pick == auto else pick
