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


def build_history(bm, lengths, prefix_len: int = 0, twins: bool = False):
    """Drive a block manager (oracle model or product) through the setup of a decode batch.

    Each sequence s ends up holding lengths[s] - 1 history positions, so that this step's append
    brings it to lengths[s].  With prefix_len > 0 a prefix sequence of prefix_len positions is
    built first, every batch sequence is forked from it and the prefix owner is then released (the
    batch's tables share its blocks).  With twins, every batch sequence is forked once more after
    its history is written and the fork is kept aside, so the block the step writes into is shared
    and the step's append must clone it.

    Returns (seqs, history) where history is a list of (owner_tag, slots) in write order: owner
    "prefix" or the batch index, with the slots its history positions were written to.
    """
    history = []
    seqs = []
    if prefix_len:
        p = bm.add_seq()
        slots = [bm.append(p)[0] for _ in range(prefix_len)]
        history.append(("prefix", slots))
        for _ in lengths:
            seqs.append(bm.fork(p))
        bm.free_seq(p)
    else:
        for _ in lengths:
            seqs.append(bm.add_seq())
    for i, (s, L) in enumerate(zip(seqs, lengths)):
        n = int(L) - 1 - prefix_len
        slots = [bm.append(s)[0] for _ in range(n)]
        history.append((i, slots))
    twin_ids = [bm.fork(s) for s in seqs] if twins else []
    return seqs, history, twin_ids
