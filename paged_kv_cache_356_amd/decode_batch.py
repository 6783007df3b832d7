"""A decode batch on the device: KV pools filled with a synthetic history, the step's metadata from
the block manager, and the calls of one decode step.

Building a batch (``DecodeBatch``):
  1. the workload's lengths and free-list order come from ``workloads``;
  2. the host block manager (pa_bm_*) runs the workload's recipe (``workloads.build_history``): it
     allocates blocks on demand, forks shared prefixes, and keeps the tables;
  3. N(0, 1) history K/V rows are written into each layer's pools with pa_reshape_and_cache (a
     prefill stand-in);
  4. the step's metadata (one appended position per sequence: slots, copy-on-write pairs, block
     tables, context lengths) is produced by the block manager and copied to the device once.

A step (``run_step``) is then pa_copy_blocks (only when the step has copy-on-write pairs; one call
for all layers), followed per layer by pa_reshape_and_cache of the new token and pa_decode_attention.
Repeating a step is idempotent: the clone is taken again from the unchanged source block and the
same token is written to the same slot.

``num_sets`` builds several independent batches of the same workload in the same pools (distinct
blocks and values), so that timing loops can rotate between them and read KV that is not already
in the caches, as successive layers of a real model would.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from . import api
from . import workloads as wl


@dataclass
class BatchSet:
    seqs: list
    history: list
    twins: list
    hist_slots: np.ndarray = None
    slots: np.ndarray = None          # this step's slot per sequence (int64)
    pairs: np.ndarray = None          # this step's copy-on-write (src, dst) rows (int32)
    tables: np.ndarray = None         # [S, max_blocks] int32
    ctx: np.ndarray = None            # [S] int32
    d_slots: torch.Tensor = None
    d_pairs: torch.Tensor = None
    d_tables: torch.Tensor = None
    d_ctx: torch.Tensor = None
    q: dict = field(default_factory=dict)       # layer -> [S, Hq, D]
    new_k: dict = field(default_factory=dict)   # layer -> [S, H, D]
    new_v: dict = field(default_factory=dict)
    hist_k: dict = field(default_factory=dict)  # layer -> [T, H, D] (only with keep_values)
    hist_v: dict = field(default_factory=dict)
    out: dict = field(default_factory=dict)     # layer -> [S, Hq, D]


def value_seed(w: wl.Workload, set_index: int, layer: int) -> int:
    return w.seed * 100003 + set_index * 1009 + layer


class DecodeBatch:
    def __init__(self, w: wl.Workload, device="cuda", num_sets: int = 1, layers=None,
                 pad_block: int = 0, keep_values: bool = False, pool_fill: int = 0,
                 lengths=None, partition_size: int | None = None, keep_layers=None,
                 contiguous: bool = False, plan: bool = True):
        self.w = w
        self.device = device
        H, D, S = w.num_kv_heads, w.head_dim, w.num_seqs
        self.lengths = wl.context_lengths(w) if lengths is None else np.asarray(lengths, np.int32)
        assert len(self.lengths) == S
        # contiguous: the free list in pool order, so that each sequence's blocks sit next to each
        # other (the control against which the block table's indirection is measured)
        self.free_order = np.arange(w.num_blocks, dtype=np.int32) if contiguous else wl.free_order(w)
        self.layers = list(range(w.num_layers)) if layers is None else list(layers)
        self.partition_size = w.partition_size if partition_size is None else partition_size
        B = w.block_size
        self.bm = api.BlockManager(w.num_blocks, B, self.free_order)

        # (2) the workload's recipe on the block manager, then (4) this step's appends
        self.sets = []
        for _ in range(num_sets):
            seqs, history, twins = wl.build_history(self.bm, self.lengths, w.prefix_len,
                                                    twins=w.prefix_len > 0)
            st = BatchSet(seqs, history, twins)
            st.hist_slots = np.concatenate([np.asarray(sl, np.int64) for _, sl in history]) \
                if history else np.zeros(0, np.int64)
            self.sets.append(st)
        for st in self.sets:
            st.slots, st.pairs = self.bm.append_batch(st.seqs)
        self.max_context_len = int(self.lengths.max()) if S else 0
        self.max_blocks = max(1, math.ceil(self.max_context_len / B))
        for st in self.sets:
            st.tables, st.ctx = self.bm.export(st.seqs, self.max_blocks, pad_block)
            st.d_slots = torch.from_numpy(st.slots).to(device)
            st.d_pairs = torch.from_numpy(np.ascontiguousarray(st.pairs, np.int32)).to(device)
            st.d_tables = torch.from_numpy(st.tables).to(device)
            st.d_ctx = torch.from_numpy(st.ctx).to(device)

        # (3) pools and history
        self.caches = {}
        for l in self.layers:
            cache = api.KVCache.allocate(w.num_blocks, H, D, w.cache_dtype, device, block_size=B)
            if pool_fill:
                cache.k_pool.fill_(pool_fill)
                cache.v_pool.fill_(pool_fill)
            self.caches[l] = cache
            for r, st in enumerate(self.sets):
                g = wl.torch_generator(value_seed(w, r, l), device)
                T = st.hist_slots.shape[0]
                hk = wl.normal((T, H, D), w.kv_dtype, g, device)
                hv = wl.normal((T, H, D), w.kv_dtype, g, device)
                st.new_k[l] = wl.normal((S, H, D), w.kv_dtype, g, device)
                st.new_v[l] = wl.normal((S, H, D), w.kv_dtype, g, device)
                st.q[l] = wl.normal((S, w.num_q_heads, D), w.q_dtype, g, device)
                st.out[l] = torch.empty_like(st.q[l])
                if w.cache_dtype == "fp8" and r == 0:
                    cache.k_scale = fp8_head_scales(hk, st.new_k[l])
                    cache.v_scale = fp8_head_scales(hv, st.new_v[l])
                if T:
                    api.pa_reshape_and_cache(cache, hk, hv,
                                             torch.from_numpy(st.hist_slots).to(device))
                if keep_values and r == 0 and (keep_layers is None or l in keep_layers):
                    # set 0's history rows, kept for checks on the host
                    st.hist_k[l], st.hist_v[l] = hk, hv
                del hk, hv
        # the shared prefix's blocks: the first prefix_len / B entries of every table (all equal)
        self.prefix_len = w.prefix_len
        self.prefix_tables = []
        if self.prefix_len:
            nb = self.prefix_len // B
            for st in self.sets:
                first = st.tables[:, :nb]
                assert (first == first[0]).all(), "the batch's tables do not share the prefix blocks"
                self.prefix_tables.append(torch.from_numpy(first[0].copy()).to(device))
        ws = api.pa_decode_workspace_bytes(S, w.num_q_heads, H, D, self.max_context_len,
                                           self.partition_size)
        if self.prefix_len:
            ws = max(ws, api.pa_decode_shared_prefix_workspace_bytes(
                S, w.num_q_heads, H, D, self.max_context_len, self.prefix_len,
                self.partition_size))
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=device)
        # use the shared-prefix decode where the workload has a prefix (run_step / run_layer)
        self.use_prefix = self.prefix_len > 0
        self.fused = False  # run_layer: one pa_decode_attention_append call instead of two
        # the decode calls take the dealing order pa_decode_plan computes from each set's lengths
        # (step metadata, like the block tables); plan=False keeps the batch order
        self.plan = plan
        self._orders = {}

    # ------------------------------------------------------------------ the step
    # The library calls of a step are prepared once per (set, layer) and replayed (api.*Call): the
    # tensors of a set never move, so only the stream is looked up per call.
    def _call(self, key, make):
        calls = self.__dict__.setdefault("_calls", {})
        c = calls.get(key)
        if c is None:
            c = calls[key] = make()
        return c

    def copy(self, set_index: int, layers=None, stream=None):
        """The step's copy-on-write clones (no call when the set has no pairs)."""
        st = self.sets[set_index]
        if not st.pairs.shape[0]:
            return
        ls = tuple(self.layers if layers is None else layers)
        self._call(("copy", set_index, ls),
                   lambda: api.CopyCall([self.caches[l] for l in ls], st.d_pairs))(stream)

    def reshape(self, set_index: int, layer: int, stream=None):
        """The step's reshape_and_cache of the new token's K/V for one layer."""
        st = self.sets[set_index]
        self._call(("reshape", set_index, layer),
                   lambda: api.ReshapeCall(self.caches[layer], st.new_k[layer], st.new_v[layer],
                                           st.d_slots))(stream)

    def run_step(self, set_index: int = 0, flags: int = api.PA_DECODE_DEFAULT, stream=None):
        self.copy(set_index, stream=stream)
        for l in self.layers:
            self.run_layer(set_index, l, flags=flags, stream=stream, copy=False)

    def run_layer(self, set_index: int, layer: int, flags: int = api.PA_DECODE_DEFAULT,
                  stream=None, copy: bool = True, reshape: bool = True):
        """One layer of the step: copy-on-write clones, then the cache write and the attention,
        as two calls (reshape_and_cache, decode) or, when `fused` is set, as one
        (pa_decode_attention_append)."""
        if copy:
            self.copy(set_index, [layer], stream)
        if self.fused and reshape:
            self.decode(set_index, layer, flags=flags, stream=stream, append=True)
            return
        if reshape:
            self.reshape(set_index, layer, stream)
        self.decode(set_index, layer, flags=flags, stream=stream)

    def plan_for(self, set_index: int, flags: int = api.PA_DECODE_DEFAULT, append: bool = False):
        """The set's dealing order and partition size for its decode calls: pa_decode_plan on the
        host copy of the set's context lengths, computed once per set and call kind.  The order
        is a device int32 [S], None with plan off or where the plan is the batch order itself
        (which the call then deals without the order's extra scan); the partition size is the
        batch's own unless that is automatic and the planner picked a larger one."""
        if not self.plan:
            return None, self.partition_size
        key = (set_index, flags, append, self.use_prefix, self.partition_size)
        if key not in self._orders:
            st = self.sets[set_index]
            w = self.w
            cache = self.caches[self.layers[0]]
            q_dtype = st.q[self.layers[0]].dtype
            order, pt = api.pa_decode_plan(
                cache, q_dtype, st.ctx, w.num_q_heads, self.max_blocks, self.max_context_len,
                self.prefix_len if self.use_prefix else 0, self.partition_size,
                flags | (api.PA_DECODE_PLAN_APPEND if append else 0), with_partition=True)
            identity = bool((order == np.arange(order.shape[0])).all())
            self._orders[key] = (None if identity else torch.from_numpy(order).to(self.device), pt)
        return self._orders[key]

    def order(self, set_index: int, flags: int = api.PA_DECODE_DEFAULT, append: bool = False):
        """The set's dealing order (plan_for)."""
        return self.plan_for(set_index, flags, append)[0]

    def call_partition(self, set_index: int = 0, flags: int = api.PA_DECODE_DEFAULT,
                       append: bool = False) -> int:
        """The partition size the set's decode calls are made with (plan_for; 0: automatic)."""
        return self.plan_for(set_index, flags, append)[1]

    def decode(self, set_index: int, layer: int, flags: int = api.PA_DECODE_DEFAULT, stream=None,
               out: torch.Tensor | None = None, append: bool = False):
        """The step's attention call for one layer (shared-prefix decode when use_prefix); with
        `append`, the fused call that also writes the step's new token."""
        st = self.sets[set_index]

        def make(o):
            pre = dict(prefix_table=self.prefix_tables[set_index], prefix_len=self.prefix_len) \
                if self.use_prefix else {}
            if append:
                pre.update(key=st.new_k[layer], value=st.new_v[layer], slot_mapping=st.d_slots)
            order, pt = self.plan_for(set_index, flags, append)
            return api.DecodeCall(o, st.q[layer], self.caches[layer], st.d_tables, st.d_ctx,
                                  self.max_context_len, self.w.scale, pt, self.workspace, flags,
                                  seq_order=order, **pre)
        if out is not None:
            make(out)(stream)
            return
        key = ("decode", set_index, layer, flags, self.use_prefix, self.partition_size, append,
               self.plan)
        self._call(key, lambda: make(st.out[layer]))(stream)

    # ------------------------------------------------------------------ accounting
    def kv_bytes_per_layer(self, unique: bool = False) -> int:
        """Algorithmic KV bytes one decode reads per layer and batch: every context position's K
        and V rows (logical), or each distinct physical slot once (unique)."""
        w = self.w
        e = 1 if w.cache_dtype == "fp8" else (4 if w.cache_dtype == "f32" else 2)
        row = 2 * w.num_kv_heads * w.head_dim * e
        if not unique:
            return int(self.lengths.astype(np.int64).sum()) * row
        st = self.sets[0]
        B = w.block_size
        slots = set()
        for s in range(w.num_seqs):
            L = int(st.ctx[s])
            for j in range(math.ceil(L / B)):
                b = int(st.tables[s, j])
                n = min(B, L - B * j)
                slots.update(b * B + t for t in range(n))
        return len(slots) * row


def fp8_head_scales(k_hist: torch.Tensor, k_new: torch.Tensor) -> torch.Tensor:
    """Per-KV-head fp32 scale amax|x| / 448 over a layer's rows, so every value fits E4M3FN."""
    amax = torch.maximum(k_hist.float().abs().amax(dim=(0, 2)) if k_hist.shape[0] else
                         torch.zeros(k_new.shape[1], device=k_new.device),
                         k_new.float().abs().amax(dim=(0, 2)))
    return (amax / 448.0).clamp_min(1e-12).contiguous()
