"""TEST INFRASTRUCTURE ONLY — the oracle's side of a decode batch.

Re-runs a batch's workload recipe on the oracle's block-manager model and rebuilds the KV pools on
the host with the oracle's replays, from the same generator outputs (history rows, new-token rows,
queries, fp8 scales) the device batch was built from, copied to the host.  Nothing here reads a
result of the HIP path: pools, tables, slots and copy pairs are all the oracle's own.  Used by the
GPU parity tests and the benchmark's CPU-baseline leg."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle.bm_model import BlockManagerModel
from paged_kv_cache_356_amd import workloads as wl

RAW_NP = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8}


def raw(t: torch.Tensor) -> np.ndarray:
    """numpy view of a tensor's raw elements on the host (float32 values, or f16/bf16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(t.dtype)


class OracleBatch:
    def __init__(self, batch, pad_block: int, pool_fill: int = 0):
        w = batch.w
        self.w = w
        self.model = BlockManagerModel(w.num_blocks, w.block_size, batch.free_order)
        self.sets = []
        for _ in batch.sets:
            seqs, history, twins = wl.build_history(self.model, batch.lengths, w.prefix_len,
                                                    twins=w.prefix_len > 0)
            self.sets.append({"seqs": seqs, "history": history})
        for st in self.sets:
            slots, pairs = self.model.append_batch(st["seqs"])
            st["slots"] = np.asarray(slots, np.int64)
            st["pairs"] = np.asarray(pairs, np.int32).reshape(-1, 2)
        for st in self.sets:
            rows, lens = self.model.export(st["seqs"], batch.max_blocks, pad_block)
            st["tables"] = np.asarray(rows, np.int32)
            st["ctx"] = np.asarray(lens, np.int32)
        self.pool_fill = pool_fill
        self.pools = {}

    def metadata_matches(self, batch) -> None:
        for st, dst in zip(self.sets, batch.sets):
            assert np.array_equal(st["slots"], dst.slots)
            assert np.array_equal(st["pairs"], np.asarray(dst.pairs).reshape(-1, 2))
            assert np.array_equal(st["tables"], dst.tables)
            assert np.array_equal(st["ctx"], dst.ctx)

    def build_pools(self, batch, layer: int, set_index: int = 0, owners=None):
        """Host pools of one layer after this step's clone and write, replayed by the oracle from
        the generator's history and new-token rows.  owners: restrict the history replay to these
        batch indices (plus the shared prefix) — enough for sampled outputs of those sequences."""
        w = self.w
        H, D = w.num_kv_heads, w.head_dim
        dt = w.cache_dtype
        B = w.block_size
        n = w.num_blocks * H * B * D
        nbytes = n * np.dtype(RAW_NP[dt]).itemsize
        if self.pool_fill:
            kp = np.full(nbytes, self.pool_fill, np.uint8).view(RAW_NP[dt])
            vp = np.full(nbytes, self.pool_fill, np.uint8).view(RAW_NP[dt])
        else:  # untouched pages of a zeroed allocation stay unmapped
            kp = np.zeros(nbytes, np.uint8).view(RAW_NP[dt])
            vp = np.zeros(nbytes, np.uint8).view(RAW_NP[dt])
        cache = batch.caches[layer]
        ks = None if cache.k_scale is None else cache.k_scale.cpu().numpy()
        vs = None if cache.v_scale is None else cache.v_scale.cpu().numpy()
        dst = batch.sets[set_index]
        st = self.sets[set_index]
        hk, hv = dst.hist_k[layer], dst.hist_v[layer]
        off = 0
        for owner, slots in st["history"]:
            m = len(slots)
            if m and (owners is None or owner == "prefix" or owner in owners):
                oracle.reshape_and_cache(kp, vp, dt, ks, vs, w.num_blocks, H, D,
                                         raw(hk[off:off + m]), raw(hv[off:off + m]), w.kv_dtype,
                                         np.asarray(slots, np.int64), B=B)
            off += m
        e = np.dtype(RAW_NP[dt]).itemsize
        if st["pairs"].shape[0]:
            oracle.copy_blocks([kp], [vp], H * B * D * e, w.num_blocks, st["pairs"])
        oracle.reshape_and_cache(kp, vp, dt, ks, vs, w.num_blocks, H, D, raw(dst.new_k[layer]),
                                 raw(dst.new_v[layer]), w.kv_dtype, st["slots"], B=B)
        self.pools[(layer, set_index)] = (kp, vp, ks, vs)
        return kp, vp

    def attention(self, batch, layer: int, set_index: int = 0, sel=None, nthreads=0):
        w = self.w
        kp, vp, ks, vs = self.pools[(layer, set_index)]
        st = self.sets[set_index]
        q = raw(batch.sets[set_index].q[layer]).reshape(w.num_seqs, -1)
        return oracle.decode_attention(q, w.q_dtype, kp, vp, w.cache_dtype, ks, vs, w.num_blocks,
                                       w.num_kv_heads, w.head_dim, st["tables"], st["ctx"],
                                       w.num_q_heads, w.scale, sel=sel, nthreads=nthreads,
                                       B=w.block_size)


def device_pool_bytes(cache) -> tuple[np.ndarray, np.ndarray]:
    return cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy()


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()
