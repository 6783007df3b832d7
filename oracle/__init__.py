"""TEST INFRASTRUCTURE ONLY — the CPU oracle for decode-step paged attention.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The product (``paged_kv_cache_356_amd``) never imports it, and it imports nothing from the
product: the two share no code.  ``oracle.c`` holds the arithmetic (fp64 attention, de-paging with
its own pool indexer, exact element decoders, the fp8 E4M3FN encoder, reshape/copy replays);
``bm_model.py`` holds the block-manager model.  This module only marshals numpy arrays into the C
functions.

Sources are cited by page title and section in ``oracle.c`` and ``bm_model.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")

F32, F16, BF16, FP8 = 0, 1, 2, 3
DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16, "fp8": FP8}
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2, FP8: 1}


def build_command(out: str = LIB_PATH) -> list[str]:
    # -O2 without -ffast-math: binary32 division and fp64 arithmetic stay IEEE.
    return ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
            "-o", out, SRC, "-lm"]


def build() -> str:
    subprocess.run(build_command(), check=True)
    return LIB_PATH


_lib = None

_p = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_f64 = ctypes.c_double
_sz = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"oracle library {LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.orc_elem_bytes.argtypes = [_i32]
        L.orc_elem_bytes.restype = _i32
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = _f64
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = _f64
        L.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_f64.restype = _f64
        L.orc_e4m3_from_f32.argtypes = [_f32]
        L.orc_e4m3_from_f32.restype = ctypes.c_uint8
        L.orc_k_index.argtypes = [_i32] * 8
        L.orc_k_index.restype = _sz
        L.orc_v_index.argtypes = [_i32] * 7
        L.orc_v_index.restype = _sz
        L.orc_gather.argtypes = [_p, _p, _p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _p, _i32, _i32]
        L.orc_gather.restype = _i32
        L.orc_decode_attention.argtypes = [_p, _p, _i32, _i64, _p, _p, _i32, _p, _p, _i32, _i32, _i32,
                                           _i32, _p, _i32, _p, _i32, _i32, _f32, _p, _p, _i32, _i32]
        L.orc_decode_attention.restype = _i32
        L.orc_attend_contiguous.argtypes = [_p, _p, _p, _p, _i32, _i32, _f64]
        L.orc_attend_contiguous.restype = None
        L.orc_reshape_and_cache.argtypes = [_p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _p, _p,
                                            _i32, _i64, _i64, _p, _i32]
        L.orc_reshape_and_cache.restype = _i32
        L.orc_copy_blocks.argtypes = [_p, _p, _i32, _sz, _i32, _p, _i32]
        L.orc_copy_blocks.restype = None
        L.orc_max_threads.argtypes = []
        L.orc_max_threads.restype = _i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None) -> int | None:
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _code(dtype) -> int:
    return DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)


# ----------------------------------------------------------------------- element decoders / codec
def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    L = lib()
    return np.array([L.orc_f16_to_f64(int(b)) for b in np.asarray(bits, np.uint16).ravel()])


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    L = lib()
    return np.array([L.orc_bf16_to_f64(int(b)) for b in np.asarray(bits, np.uint16).ravel()])


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    L = lib()
    return np.array([L.orc_e4m3_to_f64(int(c)) for c in np.asarray(codes, np.uint8).ravel()])


def e4m3_from_f32(x: np.ndarray) -> np.ndarray:
    L = lib()
    return np.array([L.orc_e4m3_from_f32(float(v)) for v in np.asarray(x, np.float32).ravel()],
                    dtype=np.uint8)


def k_index(b, h, t, i, H, D, B, dtype) -> int:
    return lib().orc_k_index(b, h, t, i, H, D, B, _code(dtype))


def v_index(b, h, t, i, H, D, B) -> int:
    return lib().orc_v_index(b, h, t, i, H, D, B)


# ----------------------------------------------------------------------------- pools / replays
def pool_elems(num_blocks: int, H: int, D: int, B: int = 16) -> int:
    return num_blocks * H * B * D


def _check_pools(k_pool, v_pool, cache_dtype, num_blocks, H, D, B):
    """The C routines index the pools by (block, head, slot, dim); refuse arrays smaller than the
    geometry they are told (a wrong block size would read past their end)."""
    need = pool_elems(num_blocks, H, D, B) * ELEM_BYTES[_code(cache_dtype)]
    for name, pool in (("k_pool", k_pool), ("v_pool", v_pool)):
        if np.asarray(pool).nbytes < need:
            raise ValueError(f"{name} holds {np.asarray(pool).nbytes} bytes, fewer than "
                             f"{num_blocks} blocks of {B} positions x {H} heads x {D} need ({need})")


def gather(k_pool, v_pool, cache_dtype, k_scale, v_scale, num_blocks, H, D, table, L, h, B=16):
    """De-page positions [0, L) of one sequence's KV head h into fp64 [L][D] arrays."""
    _check_pools(k_pool, v_pool, cache_dtype, num_blocks, H, D, B)
    kc = np.zeros((max(L, 1), D), np.float64)
    vc = np.zeros((max(L, 1), D), np.float64)
    table = np.ascontiguousarray(table, np.int32)
    ks = None if k_scale is None else np.ascontiguousarray(k_scale, np.float32)
    vs = None if v_scale is None else np.ascontiguousarray(v_scale, np.float32)
    rc = lib().orc_gather(_ptr(kc), _ptr(vc), _ptr(k_pool), _ptr(v_pool), _code(cache_dtype),
                          _ptr(ks), _ptr(vs), num_blocks, H, D, B, _ptr(table), L, h)
    if rc != 0:
        raise ValueError("block table references a block outside the pool")
    return kc[:L], vc[:L]


def attend_contiguous(q: np.ndarray, kc: np.ndarray, vc: np.ndarray, scale: float) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float64)
    kc = np.ascontiguousarray(kc, np.float64)
    vc = np.ascontiguousarray(vc, np.float64)
    L, D = kc.shape if kc.ndim == 2 else (0, q.shape[0])
    out = np.zeros(q.shape[0], np.float64)
    lib().orc_attend_contiguous(_ptr(out), _ptr(q), _ptr(kc), _ptr(vc), L, q.shape[0], scale)
    return out


def decode_attention(q, q_dtype, k_pool, v_pool, cache_dtype, k_scale, v_scale, num_blocks, H, D,
                     block_tables, context_lens, num_q_heads, scale, sel=None, nthreads=0, B=16,
                     q_stride=0):
    """fp64 decode attention.  q: raw [S][Hq*D] array (f32 values, or uint16 bits for f16/bf16).
    sel: optional (seq_idx, head_idx) int arrays; returns [len(sel)][D], else [S][Hq][D]."""
    _check_pools(k_pool, v_pool, cache_dtype, num_blocks, H, D, B)
    block_tables = np.ascontiguousarray(block_tables, np.int32)
    context_lens = np.ascontiguousarray(context_lens, np.int32)
    S, M = block_tables.shape
    ks = None if k_scale is None else np.ascontiguousarray(k_scale, np.float32)
    vs = None if v_scale is None else np.ascontiguousarray(v_scale, np.float32)
    q = np.ascontiguousarray(q)
    if sel is None:
        out = np.zeros((S, num_q_heads, D), np.float64)
        ss = hh = None
        n = -1
    else:
        ss = np.ascontiguousarray(sel[0], np.int32)
        hh = np.ascontiguousarray(sel[1], np.int32)
        n = len(ss)
        out = np.zeros((n, D), np.float64)
    rc = lib().orc_decode_attention(_ptr(out), _ptr(q), _code(q_dtype), q_stride, _ptr(k_pool),
                                    _ptr(v_pool), _code(cache_dtype), _ptr(ks), _ptr(vs),
                                    num_blocks, H, D, B, _ptr(block_tables), M,
                                    _ptr(context_lens), S, num_q_heads, float(scale), _ptr(ss),
                                    _ptr(hh), n, nthreads)
    if rc != 0:
        raise ValueError(f"oracle decode_attention failed ({rc})")
    return out


def prefill_attention(q, q_dtype, k_pool, v_pool, cache_dtype, k_scale, v_scale, num_blocks, H, D,
                      block_tables, context_lens, query_start, num_q_heads, scale, nthreads=0, B=16):
    """fp64 attention for a chunk of new tokens per sequence (a prompt, or a chunk of one).  Sequence
    s has n_s = query_start[s+1] - query_start[s] new tokens at positions L_s - n_s .. L_s - 1
    (L_s = context_lens[s]); the token at position p attends to positions 0 .. p of its sequence:
    a prompt passes through the model as one matrix whose tokens look at each other, and a token's
    K and V serve every token after it ("PagedAttention, Visualized", Parts 1 and 2).  Each token
    is therefore the decode of its own position, computed here as such.
    q: raw [num_tokens][Hq*D]; returns [num_tokens][Hq][D]."""
    block_tables = np.ascontiguousarray(block_tables, np.int32)
    context_lens = np.asarray(context_lens, np.int64)
    query_start = np.asarray(query_start, np.int64)
    S = block_tables.shape[0]
    rows, ctx = [], []
    for s in range(S):
        n = int(query_start[s + 1] - query_start[s])
        for t in range(n):
            rows.append(s)
            ctx.append(int(context_lens[s]) - n + t + 1)
    T = len(rows)
    if T == 0:
        return np.zeros((0, num_q_heads, D), np.float64)
    return decode_attention(q, q_dtype, k_pool, v_pool, cache_dtype, k_scale, v_scale, num_blocks,
                            H, D, block_tables[np.asarray(rows)], np.asarray(ctx, np.int32),
                            num_q_heads, scale, nthreads=nthreads, B=B)


def reshape_and_cache(k_pool, v_pool, cache_dtype, k_scale, v_scale, num_blocks, H, D, key, value,
                      in_dtype, slots, B=16, key_stride=None, value_stride=None):
    """In-place replay into host pools (numpy arrays of the cache's raw element type)."""
    _check_pools(k_pool, v_pool, cache_dtype, num_blocks, H, D, B)
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    slots = np.ascontiguousarray(slots, np.int64)
    T = slots.shape[0]
    ks = None if k_scale is None else np.ascontiguousarray(k_scale, np.float32)
    vs = None if v_scale is None else np.ascontiguousarray(v_scale, np.float32)
    rc = lib().orc_reshape_and_cache(_ptr(k_pool), _ptr(v_pool), _code(cache_dtype), _ptr(ks),
                                     _ptr(vs), num_blocks, H, D, B, _ptr(key), _ptr(value),
                                     _code(in_dtype),
                                     H * D if key_stride is None else key_stride,
                                     H * D if value_stride is None else value_stride,
                                     _ptr(slots), T)
    if rc != 0:
        raise ValueError("unsupported dtype combination")


def copy_blocks(k_pools, v_pools, block_bytes, num_blocks, pairs):
    pairs = np.ascontiguousarray(pairs, np.int32).reshape(-1, 2)
    n = len(k_pools)
    kp = (ctypes.c_void_p * n)(*[_ptr(a) for a in k_pools])
    vp = (ctypes.c_void_p * n)(*[_ptr(a) for a in v_pools])
    lib().orc_copy_blocks(kp, vp, n, block_bytes, num_blocks, _ptr(pairs), pairs.shape[0])


def swap_blocks(dev_pools, host_pools, block_bytes: int, num_blocks: int, num_host: int, pairs,
                to_host: bool) -> None:
    """Evicting blocks to CPU memory and bringing them back ("PagedAttention, Visualized", Part 3,
    the OS table: swapping to disk).  dev_pools / host_pools: per layer, per K and V, flat uint8
    arrays of num_blocks / num_host blocks of block_bytes.  For each (device block, host slot) pair,
    in order and for every pool, the block's bytes are copied to the slot (to_host) or back.
    Pairs naming a block or slot outside its pool are skipped."""
    pairs = np.asarray(pairs, np.int64).reshape(-1, 2)
    for d, h in pairs:
        if not (0 <= d < num_blocks and 0 <= h < num_host):
            continue
        for dev, host in zip(dev_pools, host_pools):
            ds = slice(int(d) * block_bytes, (int(d) + 1) * block_bytes)
            hs = slice(int(h) * block_bytes, (int(h) + 1) * block_bytes)
            if to_host:
                host[hs] = dev[ds]
            else:
                dev[ds] = host[hs]


def max_threads() -> int:
    return lib().orc_max_threads()
