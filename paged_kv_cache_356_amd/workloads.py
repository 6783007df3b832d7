"""Seeded synthetic inputs for the five decode workloads.

This module draws random numbers and nothing else: context lengths, the order in which physical
blocks leave the free list, and N(0, 1) query/key/value values.  It holds none of the paged-attention
arithmetic, imports nothing else from this package, and is the one module that both the product
path (benchmark) and the tests' oracle side use.

Workloads (Qwen2.5-7B-shaped heads: 28 query heads, 4 KV heads, head_dim 128 — 28 x 128 is the
model's hidden size 3584 and 4 x 128 = 512 is the per-layer K (or V) width, "PagedAttention,
Visualized" Parts 1-2; block size 16, "PagedAttention" (devoured.fyi), "PagedAttention in one
picture"):

  tiny_f32                    4 sequences, lengths {5, 16, 17, 40}, 4 query / 2 KV heads, head_dim 64, 32 blocks.
  f16_batch32                 32 sequences, lengths uniform in [128, 2048], 65,536-block pool.
  bf16_32k_batch8             8 sequences of 32,768 tokens (2,048 blocks each), split-K partitions of 512.
  f16_shared_prefix_batch256  256 sequences sharing a 1,024-token prefix (64 blocks) plus private suffixes of
      round(lognormal(ln 300, 0.8)) tokens clipped to [1, 2048].
  fp8_28layer_batch512        fp8 E4M3 cache with fp16 queries, 28 layers, 512 sequences, lengths round(lognormal(ln 600,
      1.0)) clipped to [1, 32768], 436,000 blocks per layer (about 200 GB of KV over 28 layers).

The request-length traces used by the serving benchmarks the pages quote are not available here;
the uniform and log-normal length mixes stand in for them.

Seeds: every workload uses seed 356000 + its index (tiny_f32 -> 356001 ...).  numpy's PCG64 draws the
metadata; torch's generator draws the values.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

SEED_BASE = 356000
BLOCK_SIZE = 16

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int          # physical blocks per layer pool
    cache_dtype: str         # f32 / f16 / bf16 / fp8
    q_dtype: str             # f32 / f16 / bf16
    num_layers: int = 1
    partition_size: int = 0  # 0 = library default
    prefix_len: int = 0      # shared prefix tokens
    description: str = ""
    block_size: int = BLOCK_SIZE  # token positions per block

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.head_dim)))

    @property
    def kv_dtype(self) -> str:
        """dtype of the K/V rows handed to reshape_and_cache (fp8 caches quantise f16 rows)."""
        return "f16" if self.cache_dtype == "fp8" else self.cache_dtype

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 4, 4, 2, 64, 32, "f32", "f32",
                   description="tiny fp32 paged decode, lengths {5,16,17,40}"),
    "f16_batch32": Workload("f16_batch32", 2, 32, 28, 4, 128, 65536, "f16", "f16",
                   description="Qwen2.5-7B-shaped single-layer fp16 decode, batch 32, L~U[128,2048]"),
    "bf16_32k_batch8": Workload("bf16_32k_batch8", 3, 8, 28, 4, 128, 65536, "bf16", "bf16", partition_size=512,
                   description="long-context bf16 decode, batch 8 x 32,768 tokens, partitions of 512"),
    "f16_shared_prefix_batch256": Workload("f16_shared_prefix_batch256", 4, 256, 28, 4, 128, 65536, "f16", "f16", prefix_len=1024,
                   description="shared-prefix fp16 decode, batch 256, 1,024-token shared prefix"),
    "fp8_28layer_batch512": Workload("fp8_28layer_batch512", 5, 512, 28, 4, 128, 436000, "fp8", "f16", num_layers=28,
                   description="28-layer fp8-E4M3 KV decode step, batch 512, L~lognormal(600,1)"),
}


def rng(w: Workload, stream: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([w.seed, stream]))


def context_lengths(w: Workload) -> np.ndarray:
    """Context length of every sequence AFTER this step's token is appended (int32 [S])."""
    r = rng(w, 1)
    if w.name == "tiny_f32":
        L = np.array([5, 16, 17, 40])
    elif w.name == "f16_batch32":
        L = r.integers(128, 2048, size=w.num_seqs, endpoint=True)
    elif w.name == "bf16_32k_batch8":
        L = np.full(w.num_seqs, 32768)
    elif w.name == "f16_shared_prefix_batch256":
        L = w.prefix_len + suffix_lengths(w)
    elif w.name == "fp8_28layer_batch512":
        L = np.clip(np.rint(r.lognormal(np.log(600.0), 1.0, size=w.num_seqs)), 1, 32768)
    else:
        raise KeyError(w.name)
    return np.asarray(L, np.int32)


def suffix_lengths(w: Workload) -> np.ndarray:
    """Shared-prefix workload: private suffix lengths (including this step's token), clipped to [1, 2048]."""
    r = rng(w, 2)
    s = np.clip(np.rint(r.lognormal(np.log(300.0), 0.8, size=w.num_seqs)), 1, 2048)
    return np.asarray(s, np.int32)


def free_order(w: Workload, stream: int = 3) -> np.ndarray:
    """Seeded permutation of the physical block ids: the order they leave the free list."""
    return np.asarray(rng(w, stream).permutation(w.num_blocks), np.int32)


def torch_generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, dtype: str, gen: torch.Generator, device="cpu") -> torch.Tensor:
    """N(0, 1) values drawn in fp32 and rounded to `dtype`."""
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    return x.to(TORCH_DTYPES[dtype])


def lengths_summary(L: np.ndarray) -> dict:
    return {"min": int(L.min()), "max": int(L.max()), "mean": float(L.mean()), "sum": int(L.sum())}


def build_history(bm, lengths, prefix_len: int = 0, twins: bool = False):
    """The workload's recipe of block-manager operations, run on whichever manager it is given.

    Each batch sequence s ends up holding lengths[s] - 1 positions, so this step's append brings it
    to lengths[s].  With prefix_len > 0 a prefix sequence of prefix_len positions is built first,
    every batch sequence is forked from it, and the prefix's owner is released (the batch's tables
    share its blocks).  With twins, every batch sequence is forked once more after its history is
    written and the fork is kept aside, so the block this step writes into is shared and must be
    cloned first.

    Returns (seqs, history, twin_ids); history lists (owner, slots) in write order, owner "prefix"
    or the batch index, with the slots of the positions written for that owner.
    """
    history = []
    seqs = []
    if prefix_len:
        p = bm.add_seq()
        history.append(("prefix", [bm.append(p)[0] for _ in range(prefix_len)]))
        seqs = [bm.fork(p) for _ in lengths]
        bm.free_seq(p)
    else:
        seqs = [bm.add_seq() for _ in lengths]
    for i, (s, L) in enumerate(zip(seqs, lengths)):
        n = int(L) - 1 - prefix_len
        if n < 0:
            raise ValueError(f"length {int(L)} does not cover the {prefix_len}-token prefix + 1")
        history.append((i, [bm.append(s)[0] for _ in range(n)]))
    twin_ids = [bm.fork(s) for s in seqs] if twins else []
    return seqs, history, twin_ids
