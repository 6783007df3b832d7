"""Thin Python binding of libpa.so (include/pa.h).  Argument marshalling only: every step of the
paged-attention path runs in the library's HIP kernels; torch supplies device memory and streams.

The library is loaded on first use; if it is not built, the call raises — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpa.so")

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
PA_BLOCK_SIZE = 16
PA_DECODE_DEFAULT = 0
PA_DECODE_FORCE_VALU = 1
PA_DECODE_PLAN_APPEND = 2  # pa_decode_plan only: plan for pa_decode_attention_append
PA_NOALLOC_SCRATCH_BYTES = 64 << 20  # the fixed device scratch of pa_decode_attention_noalloc
DTYPE_CODES = {"f32": PA_F32, "f16": PA_F16, "bf16": PA_BF16, "fp8": PA_FP8_E4M3}
TORCH_CODES = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
ELEM_BYTES = {PA_F32: 4, PA_F16: 2, PA_BF16: 2, PA_FP8_E4M3: 1}

STATUS = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_UNSUPPORTED",
          -4: "PA_ERR_WORKSPACE", -5: "PA_ERR_ALIAS", -6: "PA_ERR_LAUNCH", -7: "PA_ERR_NO_BLOCKS",
          -8: "PA_ERR_STATE"}

# Every symbol include/*.h declares.
EXPORTS = [
    "pa_calibrate_read",
    "pa_pool_bytes", "pa_reshape_and_cache", "pa_decode_auto_partition",
    "pa_decode_workspace_bytes", "pa_decode_attention", "pa_decode_attention_shared_prefix",
    "pa_decode_attention_append", "pa_decode_attention_noalloc",
    "pa_decode_shared_prefix_workspace_bytes", "pa_copy_blocks", "pa_check_copy_pairs",
    "pa_check_slots", "pa_check_context_lens", "pa_check_seq_order", "pa_decode_plan",
    "pa_set_debug", "pa_debug_enabled",
    "pa_prefill_attention", "pa_swap_blocks", "pa_bm_set_host_blocks", "pa_bm_swap_out",
    "pa_bm_swap_in",
    "pa_bm_num_free_host", "pa_bm_is_swapped",
    "pa_status_string", "pa_last_error", "pa_bm_create", "pa_bm_destroy", "pa_bm_add_seq",
    "pa_bm_fork", "pa_bm_append", "pa_bm_append_batch", "pa_bm_free_seq", "pa_bm_refcount",
    "pa_bm_num_free", "pa_bm_seq_len", "pa_bm_block_table", "pa_bm_export",
]


class PaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class pa_cache(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("cache_dtype", ctypes.c_int32)]


_lib = None
_vp, _i32, _i64, _u32, _f32, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                    ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t)
_cp = ctypes.POINTER(pa_cache)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (python -m paged_kv_cache_356_amd.build); "
                               "there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "pa_pool_bytes": (_sz, [_cp]),
            "pa_calibrate_read": (_i32, [_vp, _vp, _i64, _vp, _i64, _vp, _vp]),
            "pa_reshape_and_cache": (_i32, [_cp, _vp, _vp, _i32, _i64, _i64, _vp, _i32, _vp]),
            "pa_decode_auto_partition": (_i32, [_i32, _i32, _i32]),
            "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
            "pa_decode_attention": (_i32, [_vp, _vp, _i32, _i64, _cp, _vp, _i32, _vp, _vp, _i32,
                                           _i32, _i32, _f32, _i32, _vp, _sz, _u32, _vp]),
            "pa_decode_attention_shared_prefix": (_i32, [_vp, _vp, _i32, _i64, _cp, _vp, _i32, _vp,
                                                          _vp, _i32, _i32, _i32, _f32, _vp, _i32,
                                                          _i32, _vp, _sz, _u32, _vp]),
            "pa_decode_attention_append": (_i32, [_vp, _vp, _i32, _i64, _cp, _vp, _vp, _i64, _i64,
                                                   _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _f32,
                                                   _vp, _i32, _i32, _vp, _sz, _u32, _vp]),
            "pa_decode_plan": (_i32, [_cp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _u32,
                                      _vp, _vp, _vp]),
            "pa_check_seq_order": (_i32, [_vp, _i32]),
            "pa_decode_attention_noalloc": (_i32, [_vp, _vp, _i32, _i64, _cp, _vp, _i32, _vp,
                                                    _i32, _i32, _i32, _f32, _i32, _u32, _vp]),
            "pa_decode_shared_prefix_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32,
                                                              _i32]),
            "pa_copy_blocks": (_i32, [_cp, _i32, _vp, _i32, _vp]),
            "pa_check_copy_pairs": (_i32, [_vp, _i32, _i32]),
            "pa_check_slots": (_i32, [_vp, _i32, _i32, _i32]),
            "pa_check_context_lens": (_i32, [_vp, _i32, _i32]),
            "pa_set_debug": (None, [ctypes.c_int]),
            "pa_debug_enabled": (ctypes.c_int, []),
            "pa_swap_blocks": (_i32, [_cp, _i32, _vp, _vp, _i32, _vp, _i32, _i32, _vp]),
            "pa_prefill_attention": (_i32, [_vp, _vp, _i32, _i64, _cp, _vp, _i32, _vp, _vp, _i32,
                                            _i32, _i32, _i32, _i32, _f32, _vp]),
            "pa_bm_set_host_blocks": (_i32, [_vp, _i32]),
            "pa_bm_swap_out": (_i32, [_vp, _i32, _vp, _i32, _vp]),
            "pa_bm_swap_in": (_i32, [_vp, _i32, _vp, _i32, _vp]),
            "pa_bm_num_free_host": (_i32, [_vp]),
            "pa_bm_is_swapped": (_i32, [_vp, _i32]),
            "pa_status_string": (ctypes.c_char_p, [_i32]),
            "pa_last_error": (ctypes.c_char_p, []),
            "pa_bm_create": (_vp, [_i32, _i32, _vp]),
            "pa_bm_destroy": (None, [_vp]),
            "pa_bm_add_seq": (_i32, [_vp, _vp]),
            "pa_bm_fork": (_i32, [_vp, _i32, _vp]),
            "pa_bm_append": (_i32, [_vp, _i32, _vp, _vp, _vp]),
            "pa_bm_append_batch": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp]),
            "pa_bm_free_seq": (_i32, [_vp, _i32]),
            "pa_bm_refcount": (_i32, [_vp, _i32]),
            "pa_bm_num_free": (_i32, [_vp]),
            "pa_bm_seq_len": (_i32, [_vp, _i32]),
            "pa_bm_block_table": (_i32, [_vp, _i32, _vp, _i32, _vp]),
            "pa_bm_export": (_i32, [_vp, _vp, _i32, _vp, _i32, _i32, _vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise PaError(status, lib().pa_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.data_ptr()
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return int(t)


_have_gpu = None


def _stream(stream) -> int | None:
    """The hipStream_t to enqueue on: torch's current stream when `stream` is None."""
    global _have_gpu
    if stream is None:
        if _have_gpu is None:
            _have_gpu = torch.cuda.is_available()
        if not _have_gpu:
            return None
        return torch._C._cuda_getCurrentRawStream(torch._C._cuda_getDevice())
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# --------------------------------------------------------------------------- KV cache (one layer)
@dataclass
class KVCache:
    """One layer's pools (raw bytes in the library's layout) plus, for fp8, per-head scales."""
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    num_blocks: int
    num_kv_heads: int
    head_dim: int
    cache_dtype: int
    k_scale: torch.Tensor | None = None
    v_scale: torch.Tensor | None = None
    block_size: int = PA_BLOCK_SIZE

    @staticmethod
    def allocate(num_blocks, num_kv_heads, head_dim, cache_dtype, device="cuda", k_scale=None,
                 v_scale=None, block_size=PA_BLOCK_SIZE) -> "KVCache":
        code = DTYPE_CODES[cache_dtype] if isinstance(cache_dtype, str) else int(cache_dtype)
        n = pool_bytes(num_blocks, num_kv_heads, head_dim, code, block_size)
        return KVCache(torch.zeros(n, dtype=torch.uint8, device=device),
                       torch.zeros(n, dtype=torch.uint8, device=device), num_blocks, num_kv_heads,
                       head_dim, code, k_scale, v_scale, block_size)

    def struct(self) -> pa_cache:
        """The pa_cache of this layer (built once; rebuilt if a pool tensor was replaced)."""
        key = (_ptr(self.k_pool), _ptr(self.v_pool), _ptr(self.k_scale), _ptr(self.v_scale),
               self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim,
               self.cache_dtype)
        c = self.__dict__.get("_c")
        if c is None or self.__dict__.get("_key") != key:
            c = pa_cache(*key)
            self.__dict__["_c"], self.__dict__["_key"] = c, key
        return c


def pool_bytes(num_blocks, num_kv_heads, head_dim, cache_dtype, block_size=PA_BLOCK_SIZE) -> int:
    c = pa_cache(None, None, None, None, num_blocks, block_size, num_kv_heads, head_dim,
                 int(cache_dtype))
    n = lib().pa_pool_bytes(ctypes.byref(c))
    if n == 0 and num_blocks > 0:
        raise PaError(-2, "invalid cache description")
    return n


# --------------------------------------------------------------------------- kernels
def pa_calibrate_read(k_pool: torch.Tensor, v_pool: torch.Tensor, tile_bytes: int,
                      tiles: torch.Tensor | None, num_tiles: int, sink: torch.Tensor,
                      stream=None) -> None:
    """The read-bandwidth reference (include/pa_calibrate.h): read the listed tiles of both pools;
    sink holds at least ceil(num_tiles / 4) words."""
    _check(lib().pa_calibrate_read(_ptr(k_pool), _ptr(v_pool), int(tile_bytes), _ptr(tiles),
                                   int(num_tiles), _ptr(sink), _stream(stream)))


class ReshapeCall:
    """pa_reshape_and_cache with every argument but the stream fixed: the checks and conversions
    are done once, when the call is made, for loops that repeat it."""

    def __init__(self, cache: KVCache, key: torch.Tensor, value: torch.Tensor,
                 slot_mapping: torch.Tensor):
        assert slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous()
        T = slot_mapping.shape[0]
        assert key.dtype == value.dtype and key.shape[0] == T and value.shape[0] == T
        for t in (key, value):  # rows [num_kv_heads, head_dim] contiguous, strided along T
            assert t.dim() == 3 and t.stride(2) == 1 and t.stride(1) == t.shape[2]
        self._keep = (cache, key, value, slot_mapping)
        self._args = (ctypes.byref(cache.struct()), _ptr(key), _ptr(value),
                      TORCH_CODES[key.dtype], key.stride(0) if T else 0,
                      value.stride(0) if T else 0, _ptr(slot_mapping), T)
        self._fn = lib().pa_reshape_and_cache

    def __call__(self, stream=None) -> None:
        _check(self._fn(*self._args, _stream(stream)))


def pa_reshape_and_cache(cache: KVCache, key: torch.Tensor, value: torch.Tensor,
                         slot_mapping: torch.Tensor, stream=None) -> None:
    """key/value: [T, num_kv_heads, head_dim] (rows may be strided along T); slot_mapping int64 [T]."""
    ReshapeCall(cache, key, value, slot_mapping)(stream)


def pa_decode_auto_partition(num_seqs, num_kv_heads, max_context_len) -> int:
    return lib().pa_decode_auto_partition(num_seqs, num_kv_heads, max_context_len)


def pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                              partition_size=0) -> int:
    return lib().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           max_context_len, partition_size)


class DecodeCall:
    """pa_decode_attention, or pa_decode_attention_shared_prefix when prefix_table is given, or
    pa_decode_attention_append when the new tokens (key, value: [S, num_kv_heads, head_dim], rows
    strided along S; slot_mapping int64 [S]) are given, with every argument but the stream fixed:
    the checks and conversions are done once, when the call is made, for loops that repeat it (a
    decode step per layer)."""

    def __init__(self, out: torch.Tensor, query: torch.Tensor, cache: KVCache,
                 block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                 scale: float, partition_size: int = 0, workspace: torch.Tensor | None = None,
                 flags: int = PA_DECODE_DEFAULT, prefix_table: torch.Tensor | None = None,
                 prefix_len: int = 0, key: torch.Tensor | None = None,
                 value: torch.Tensor | None = None, slot_mapping: torch.Tensor | None = None,
                 seq_order: torch.Tensor | None = None):
        S, Hq, D = query.shape
        assert out.shape == query.shape and out.dtype == query.dtype and out.is_contiguous()
        assert query.stride(2) == 1 and query.stride(1) == D  # rows contiguous, strided along S
        assert block_tables.dtype == torch.int32 and block_tables.is_contiguous()
        assert context_lens.dtype == torch.int32 and context_lens.is_contiguous()
        if seq_order is not None:
            assert seq_order.dtype == torch.int32 and seq_order.is_contiguous()
            assert seq_order.shape == (S,)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        head = (_ptr(out), _ptr(query), TORCH_CODES[query.dtype], query.stride(0) if S else 0,
                ctypes.byref(cache.struct()), _ptr(block_tables), block_tables.shape[1],
                _ptr(context_lens), _ptr(seq_order), S, Hq, int(max_context_len), float(scale))
        tail = (int(partition_size), _ptr(workspace), ws_bytes, int(flags))
        self._keep = (out, query, cache, block_tables, context_lens, workspace, prefix_table, key,
                      value, slot_mapping, seq_order)
        if key is not None:
            assert value is not None and slot_mapping is not None
            assert key.dtype == query.dtype and value.dtype == query.dtype
            assert key.shape[0] == S and value.shape[0] == S and slot_mapping.shape[0] == S
            for t in (key, value):
                assert t.stride(-1) == 1 and t[0].is_contiguous()
            assert slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous()
            if prefix_table is not None:
                assert prefix_table.dtype == torch.int32 and prefix_table.is_contiguous()
            self._fn = lib().pa_decode_attention_append
            self._args = head[:5] + (_ptr(key), _ptr(value), key.stride(0) if S else 0,
                                     value.stride(0) if S else 0, _ptr(slot_mapping)) + head[5:] + \
                (_ptr(prefix_table), int(prefix_len) if prefix_table is not None else 0) + tail
        elif prefix_table is None:
            self._fn = lib().pa_decode_attention
            self._args = head + tail
        else:
            assert prefix_table.dtype == torch.int32 and prefix_table.is_contiguous()
            self._fn = lib().pa_decode_attention_shared_prefix
            self._args = head + (_ptr(prefix_table), int(prefix_len)) + tail

    def __call__(self, stream=None) -> None:
        _check(self._fn(*self._args, _stream(stream)))


def pa_decode_attention(out: torch.Tensor, query: torch.Tensor, cache: KVCache,
                        block_tables: torch.Tensor, context_lens: torch.Tensor,
                        max_context_len: int, scale: float, partition_size: int = 0,
                        workspace: torch.Tensor | None = None, flags: int = PA_DECODE_DEFAULT,
                        stream=None, seq_order: torch.Tensor | None = None) -> None:
    """out, query: [S, num_q_heads, head_dim] (query rows may be strided along S);
    block_tables int32 [S, max_blocks_per_seq]; context_lens int32 [S]; seq_order: None or device
    int32 [S], a permutation of the sequences (the dealing order, pa_decode_plan)."""
    DecodeCall(out, query, cache, block_tables, context_lens, max_context_len, scale,
               partition_size, workspace, flags, seq_order=seq_order)(stream)


def pa_decode_plan(cache: KVCache, q_dtype: torch.dtype, context_lens, num_q_heads: int,
                   max_blocks_per_seq: int, max_context_len: int, prefix_len: int = 0,
                   partition_size: int = 0, flags: int = PA_DECODE_DEFAULT,
                   with_round: bool = False, with_partition: bool = False):
    """The dealing order pa_decode_plan computes from the host's context lengths (a sequence of
    ints): an int32 numpy array [S]; with_round also returns the items per round, with_partition
    the partition size to make the call with (order, [round], [partition])."""
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    S = int(lens.shape[0])
    order = np.empty(S, np.int32)
    rnd = ctypes.c_int32(0)
    pt = ctypes.c_int32(0)
    _check(lib().pa_decode_plan(ctypes.byref(cache.struct()), TORCH_CODES[q_dtype], _ptr(lens), S,
                                int(num_q_heads), int(max_blocks_per_seq), int(max_context_len),
                                int(prefix_len), int(partition_size), int(flags), _ptr(order),
                                ctypes.byref(rnd), ctypes.byref(pt)))
    out = (order,) + ((rnd.value,) if with_round else ()) + ((pt.value,) if with_partition else ())
    return out if len(out) > 1 else order


def pa_decode_attention_noalloc(out: torch.Tensor, query: torch.Tensor, cache: KVCache,
                                block_tables: torch.Tensor, context_lens: torch.Tensor,
                                max_context_len: int, scale: float, partition_size: int = 0,
                                flags: int = PA_DECODE_DEFAULT, stream=None) -> None:
    """pa_decode_attention with the partials in the library's fixed device scratch (no workspace
    argument, nothing allocated by the call)."""
    S, Hq, D = query.shape
    assert out.shape == query.shape and out.dtype == query.dtype and out.is_contiguous()
    assert query.stride(2) == 1 and query.stride(1) == D
    assert block_tables.dtype == torch.int32 and block_tables.is_contiguous()
    assert context_lens.dtype == torch.int32 and context_lens.is_contiguous()
    _check(lib().pa_decode_attention_noalloc(
        _ptr(out), _ptr(query), TORCH_CODES[query.dtype], query.stride(0) if S else 0,
        ctypes.byref(cache.struct()), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        S, Hq, int(max_context_len), float(scale), int(partition_size), int(flags),
        _stream(stream)))


def pa_decode_attention_append(out: torch.Tensor, query: torch.Tensor, cache: KVCache,
                               key: torch.Tensor, value: torch.Tensor, slot_mapping: torch.Tensor,
                               block_tables: torch.Tensor, context_lens: torch.Tensor,
                               max_context_len: int, scale: float,
                               prefix_table: torch.Tensor | None = None, prefix_len: int = 0,
                               partition_size: int = 0, workspace: torch.Tensor | None = None,
                               flags: int = PA_DECODE_DEFAULT, stream=None,
                               seq_order: torch.Tensor | None = None) -> None:
    """pa_reshape_and_cache of each sequence's new token (key, value [S, num_kv_heads, head_dim] in
    the query dtype, slot_mapping int64 [S]: the slot of position context_lens[s] - 1) followed by
    the decode (plain, or shared-prefix when prefix_table is given), in one call."""
    DecodeCall(out, query, cache, block_tables, context_lens, max_context_len, scale,
               partition_size, workspace, flags, prefix_table, prefix_len, key, value,
               slot_mapping, seq_order)(stream)


def pa_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                            max_context_len, prefix_len,
                                            partition_size=0) -> int:
    return lib().pa_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                         head_dim, max_context_len, prefix_len,
                                                         partition_size)


def pa_decode_attention_shared_prefix(out: torch.Tensor, query: torch.Tensor, cache: KVCache,
                                      block_tables: torch.Tensor, context_lens: torch.Tensor,
                                      max_context_len: int, scale: float,
                                      prefix_table: torch.Tensor, prefix_len: int,
                                      partition_size: int = 0,
                                      workspace: torch.Tensor | None = None,
                                      flags: int = PA_DECODE_DEFAULT, stream=None,
                                      seq_order: torch.Tensor | None = None) -> None:
    """pa_decode_attention for a batch sharing its first prefix_len positions (the blocks in
    prefix_table, device int32 [prefix_len / 16])."""
    DecodeCall(out, query, cache, block_tables, context_lens, max_context_len, scale,
               partition_size, workspace, flags, prefix_table, prefix_len,
               seq_order=seq_order)(stream)


class PrefillCall:
    """pa_prefill_attention with every argument but the stream fixed (checks and conversions done
    once).  out, query: [num_tokens, num_q_heads, head_dim] (query rows may be strided);
    query_start: device int32 [num_seqs + 1]."""

    def __init__(self, out: torch.Tensor, query: torch.Tensor, cache: KVCache,
                 block_tables: torch.Tensor, context_lens: torch.Tensor,
                 query_start: torch.Tensor, max_query_len: int, max_context_len: int,
                 scale: float):
        T, Hq, D = query.shape
        assert out.shape == query.shape and out.dtype == query.dtype and out.is_contiguous()
        assert query.stride(2) == 1 and query.stride(1) == D
        assert block_tables.dtype == torch.int32 and block_tables.is_contiguous()
        assert context_lens.dtype == torch.int32 and context_lens.is_contiguous()
        assert query_start.dtype == torch.int32 and query_start.is_contiguous()
        S = block_tables.shape[0]
        assert query_start.shape[0] == S + 1 and context_lens.shape[0] == S
        self._keep = (out, query, cache, block_tables, context_lens, query_start)
        self._args = (_ptr(out), _ptr(query), TORCH_CODES[query.dtype], query.stride(0) if T else 0,
                      ctypes.byref(cache.struct()), _ptr(block_tables), block_tables.shape[1],
                      _ptr(context_lens), _ptr(query_start), S, T, Hq, int(max_query_len),
                      int(max_context_len), float(scale))
        self._fn = lib().pa_prefill_attention

    def __call__(self, stream=None) -> None:
        _check(self._fn(*self._args, _stream(stream)))


def pa_prefill_attention(out, query, cache, block_tables, context_lens, query_start,
                         max_query_len: int, max_context_len: int, scale: float,
                         stream=None) -> None:
    PrefillCall(out, query, cache, block_tables, context_lens, query_start, max_query_len,
                max_context_len, scale)(stream)


class CopyCall:
    """pa_copy_blocks with every argument but the stream fixed (checks and conversions done once)."""

    def __init__(self, caches: list[KVCache], block_pairs: torch.Tensor):
        assert block_pairs.dtype == torch.int32 and block_pairs.is_contiguous()
        arr = (pa_cache * len(caches))(*[c.struct() for c in caches])
        self._keep = (caches, block_pairs, arr)
        self._args = (arr, len(caches), _ptr(block_pairs), block_pairs.shape[0])
        self._fn = lib().pa_copy_blocks

    def __call__(self, stream=None) -> None:
        _check(self._fn(*self._args, _stream(stream)))


def pa_copy_blocks(caches: list[KVCache], block_pairs: torch.Tensor, stream=None) -> None:
    """block_pairs: device int32 [P, 2] of (src, dst); every layer in `caches` is copied."""
    CopyCall(caches, block_pairs)(stream)


class HostPools:
    """Pinned host memory for swapped-out blocks: per layer, a K and a V pool of num_host_blocks
    blocks laid out as in the layer's device pool."""

    def __init__(self, caches: list[KVCache], num_host_blocks: int):
        c = caches[0]
        self.num_host_blocks = num_host_blocks
        self.block_bytes = pool_bytes(c.num_blocks, c.num_kv_heads, c.head_dim,
                                      c.cache_dtype) // max(c.num_blocks, 1)
        n = max(num_host_blocks * self.block_bytes, 1)
        self.k = [torch.empty(n, dtype=torch.uint8, pin_memory=True) for _ in caches]
        self.v = [torch.empty(n, dtype=torch.uint8, pin_memory=True) for _ in caches]


class SwapCall:
    """pa_swap_blocks with every argument but the stream fixed (checks and conversions done once)."""

    def __init__(self, caches: list[KVCache], host: HostPools, block_pairs: torch.Tensor,
                 to_host: bool):
        assert block_pairs.dtype == torch.int32 and block_pairs.is_contiguous()
        assert len(host.k) == len(caches)
        arr = (pa_cache * len(caches))(*[c.struct() for c in caches])
        hk = (ctypes.c_void_p * len(caches))(*[_ptr(t) for t in host.k])
        hv = (ctypes.c_void_p * len(caches))(*[_ptr(t) for t in host.v])
        self._keep = (caches, host, block_pairs, arr, hk, hv)
        self._args = (arr, len(caches), hk, hv, host.num_host_blocks, _ptr(block_pairs),
                      block_pairs.shape[0], int(bool(to_host)))
        self._fn = lib().pa_swap_blocks

    def __call__(self, stream=None) -> None:
        _check(self._fn(*self._args, _stream(stream)))


def pa_swap_blocks(caches: list[KVCache], host: HostPools, block_pairs: torch.Tensor,
                   to_host: bool, stream=None) -> None:
    """block_pairs: int32 [P, 2] of (device block, host slot) in device or pinned host memory; every
    layer in `caches` is copied to its host pools (to_host) or back."""
    SwapCall(caches, host, block_pairs, to_host)(stream)


def pa_check_slots(slots: np.ndarray, num_blocks: int, block_size: int = PA_BLOCK_SIZE) -> None:
    slots = np.ascontiguousarray(slots, np.int64)
    _check(lib().pa_check_slots(_ptr(slots), slots.shape[0], num_blocks, block_size))


def pa_check_context_lens(context_lens: np.ndarray, max_context_len: int) -> None:
    lens = np.ascontiguousarray(context_lens, np.int32)
    _check(lib().pa_check_context_lens(_ptr(lens), lens.shape[0], int(max_context_len)))


def pa_check_seq_order(seq_order: np.ndarray) -> None:
    order = np.ascontiguousarray(seq_order, np.int32)
    _check(lib().pa_check_seq_order(_ptr(order), order.shape[0]))


def pa_set_debug(on: bool) -> None:
    """The library's PA_DEBUG checks on or off, process-wide."""
    lib().pa_set_debug(1 if on else 0)


def pa_debug_enabled() -> bool:
    return bool(lib().pa_debug_enabled())


def pa_check_copy_pairs(pairs: np.ndarray, num_blocks: int) -> None:
    pairs = np.ascontiguousarray(pairs, np.int32).reshape(-1, 2)
    _check(lib().pa_check_copy_pairs(_ptr(pairs), pairs.shape[0], num_blocks))


# --------------------------------------------------------------------------- block manager
class BlockManager:
    """Host block manager (pa_bm_*): free list, reference counts, block tables, copy-on-write."""

    def __init__(self, num_blocks: int, block_size: int = PA_BLOCK_SIZE, free_order=None):
        self.num_blocks, self.block_size = num_blocks, block_size
        fo = None if free_order is None else np.ascontiguousarray(free_order, np.int32)
        self._h = lib().pa_bm_create(num_blocks, block_size, _ptr(fo))
        if not self._h:
            raise PaError(-2, "pa_bm_create rejected its arguments")

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.pa_bm_destroy(h)
            self._h = None

    def add_seq(self) -> int:
        out = ctypes.c_int32()
        _check(lib().pa_bm_add_seq(self._h, ctypes.byref(out)))
        return out.value

    def fork(self, parent: int) -> int:
        out = ctypes.c_int32()
        _check(lib().pa_bm_fork(self._h, parent, ctypes.byref(out)))
        return out.value

    def append(self, seq: int):
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pa_bm_append(self._h, seq, ctypes.byref(slot), ctypes.byref(src),
                                  ctypes.byref(dst)))
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def append_batch(self, seqs):
        seqs = np.ascontiguousarray(seqs, np.int32)
        n = seqs.shape[0]
        slots = np.zeros(n, np.int64)
        pairs = np.zeros((max(n, 1), 2), np.int32)
        npairs = ctypes.c_int32()
        _check(lib().pa_bm_append_batch(self._h, _ptr(seqs), n, _ptr(slots), _ptr(pairs),
                                        ctypes.byref(npairs)))
        return slots, pairs[: npairs.value].copy()

    def append_many(self, seq: int, n: int) -> np.ndarray:
        """n appends to one sequence (history fill); returns their slots."""
        out = np.zeros(n, np.int64)
        for i in range(n):
            out[i] = self.append(seq)[0]
        return out

    def free_seq(self, seq: int) -> None:
        _check(lib().pa_bm_free_seq(self._h, seq))

    def set_host_blocks(self, n: int) -> None:
        _check(lib().pa_bm_set_host_blocks(self._h, n))

    def _swap(self, fn, seq: int) -> np.ndarray:
        cap = max(self.seq_len(seq), 0) // self.block_size + 1
        pairs = np.zeros((cap, 2), np.int32)
        n = ctypes.c_int32()
        _check(fn(self._h, seq, _ptr(pairs), cap, ctypes.byref(n)))
        return pairs[: n.value].copy()

    def swap_out(self, seq: int) -> np.ndarray:
        """Evict seq's unshared blocks to host slots; returns the (device block, host slot) pairs."""
        return self._swap(lib().pa_bm_swap_out, seq)

    def swap_in(self, seq: int) -> np.ndarray:
        """Bring seq back into fresh device blocks; returns the (device block, host slot) pairs."""
        return self._swap(lib().pa_bm_swap_in, seq)

    def num_free_host(self) -> int:
        return lib().pa_bm_num_free_host(self._h)

    def is_swapped(self, seq: int) -> int:
        return lib().pa_bm_is_swapped(self._h, seq)

    def refcount(self, block: int) -> int:
        return lib().pa_bm_refcount(self._h, block)

    def num_free(self) -> int:
        return lib().pa_bm_num_free(self._h)

    def seq_len(self, seq: int) -> int:
        return lib().pa_bm_seq_len(self._h, seq)

    def table(self, seq: int) -> list[int]:
        n = ctypes.c_int32()
        _check(lib().pa_bm_block_table(self._h, seq, None, 0, ctypes.byref(n)))
        out = np.zeros(max(n.value, 1), np.int32)
        _check(lib().pa_bm_block_table(self._h, seq, _ptr(out), n.value, ctypes.byref(n)))
        return out[: n.value].tolist()

    def export(self, seqs, max_blocks: int, pad: int = 0):
        seqs = np.ascontiguousarray(seqs, np.int32)
        tables = np.zeros((seqs.shape[0], max_blocks), np.int32)
        lens = np.zeros(seqs.shape[0], np.int32)
        _check(lib().pa_bm_export(self._h, _ptr(seqs), seqs.shape[0], _ptr(tables), max_blocks,
                                  pad, _ptr(lens)))
        return tables, lens
