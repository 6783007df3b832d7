"""Pins for the CPU oracle: each check ties it to something other than itself — library routines
(numpy / torch dtype conversions, torch's scaled_dot_product_attention), closed forms, the
invariances the pages state, and the worked example the pages print.  CPU only."""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tests.helpers import RAW_NP, host_pool, nan_bits, raw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()


# ------------------------------------------------------------------------ element decoders
def test_f16_decoder_matches_numpy_all_codes():
    codes = np.arange(65536, dtype=np.uint16)
    ours = oracle.f16_to_f64(codes)
    ref = codes.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_bf16_decoder_matches_torch_all_codes():
    codes = np.arange(65536, dtype=np.uint16)
    ours = oracle.bf16_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_e4m3_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # format facts: largest finite 448, smallest subnormal 2^-9, smallest normal 2^-6, one = 0x38
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert ours[0x38] == 1.0 and np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert np.signbit(ours[0x80]) and ours[0x80] == 0.0


# ------------------------------------------------------------------------ fp8 encoder
def _finite_codes():
    return [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_e4m3_encoder_round_trips_every_finite_code():
    codes = np.array(_finite_codes(), np.uint8)
    vals = oracle.e4m3_to_f64(codes).astype(np.float32)
    back = oracle.e4m3_from_f32(vals)
    assert np.array_equal(back, codes)


def test_e4m3_encoder_ties_go_to_even_and_neighbours_to_nearest():
    pos = np.arange(0, 0x7E, dtype=np.uint8)
    lo = oracle.e4m3_to_f64(pos)
    hi = oracle.e4m3_to_f64(pos + 1)
    mid = ((lo + hi) / 2).astype(np.float32)  # exact in binary32
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    got = oracle.e4m3_from_f32(mid)
    want = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    below = np.nextafter(mid, np.float32(-np.inf), dtype=np.float32)
    above = np.nextafter(mid, np.float32(np.inf), dtype=np.float32)
    assert np.array_equal(oracle.e4m3_from_f32(below), pos)
    assert np.array_equal(oracle.e4m3_from_f32(above), (pos + 1).astype(np.uint8))
    # negative side mirrors with the sign bit
    assert np.array_equal(oracle.e4m3_from_f32(-mid), want | 0x80)


def test_e4m3_encoder_matches_torch_inside_range():
    g = np.random.default_rng(7)
    x = np.concatenate([
        g.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)
    ] + [g.uniform(-447.9, 447.9, 20000)]).astype(np.float32)
    x = x[np.abs(x) < 448]
    ours = oracle.e4m3_from_f32(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encoder_saturates_and_keeps_nan():
    big = np.array([448.0, 448.5, 463.9, 464.0, 500.0, 1e30, np.inf], np.float32)
    assert np.all(oracle.e4m3_from_f32(big) == 0x7E)
    assert np.all(oracle.e4m3_from_f32(-big) == 0xFE)
    assert oracle.e4m3_from_f32(np.array([np.nan], np.float32))[0] == 0x7F
    assert oracle.e4m3_from_f32(np.array([-np.nan], np.float32))[0] == 0xFF
    assert oracle.e4m3_from_f32(np.array([-0.0], np.float32))[0] == 0x80
    assert oracle.e4m3_from_f32(np.array([2.0 ** -11], np.float32))[0] == 0x00  # below half the
    assert oracle.e4m3_from_f32(np.array([2.0 ** -10 * 1.01], np.float32))[0] == 0x01  # 2^-9 step


# ------------------------------------------------------------------------ pool layout
def test_pool_indexer_hand_values():
    # Worked by hand from the layout description (H=2 KV heads, D=64, B=16):
    # f16 (E=8), element (b=3, h=1, t=5, i=19): tile 7*1024 = 7168; vector (19//8)=2 -> 2*16+5 = 37;
    # 37*8 + 19%8 = 299  ->  7467.
    assert oracle.k_index(3, 1, 5, 19, 2, 64, 16, "f16") == 7467
    # f32 (E=4), last element of tile 0: vector 15, token 15 -> (15*16+15)*4 + 3 = 1023.
    assert oracle.k_index(0, 0, 15, 63, 2, 64, 16, "f32") == 1023
    # fp8 (E=16), (b=1, h=0, t=2, i=17): tile 2*1024 = 2048; vector 1 -> 1*16+2 = 18; 18*16+1 = 289.
    assert oracle.k_index(1, 0, 2, 17, 2, 64, 16, "fp8") == 2337
    # V tile is transposed: (b=3, h=1, t=5, i=19) -> 7168 + 19*16 + 5 = 7477.
    assert oracle.v_index(3, 1, 5, 19, 2, 64, 16) == 7477


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
def test_pool_indexer_is_a_bijection_on_each_tile(dtype):
    H, D, B = 2, 64, 16
    for (b, h) in [(0, 0), (2, 1)]:
        ks = {oracle.k_index(b, h, t, i, H, D, B, dtype) for t in range(B) for i in range(D)}
        vs = {oracle.v_index(b, h, t, i, H, D, B) for t in range(B) for i in range(D)}
        base = (b * H + h) * B * D
        assert ks == set(range(base, base + B * D)) == vs


# ------------------------------------------------------------------------ worked example (paging)
def test_lesson06_worked_example():
    from oracle.bm_model import BlockManagerModel
    gold = json.load(open(os.path.join(GOLDEN, "lesson06_paging_example.json")))
    B = gold["block_size"]
    bm = BlockManagerModel(gold["num_pages"], B)
    A, Bq, C, D = (bm.add_seq() for _ in range(4))
    a_slots = []

    def put(seq, n, out=None):
        for _ in range(n):
            s, cow = bm.append(seq)
            assert cow is None
            if out is not None:
                out.append(s)

    # Interleaved growth reproduces the diagram's page assignment; D is a request that finishes.
    put(A, 4, a_slots); put(Bq, 4); put(D, 4); put(A, 4, a_slots); put(C, 4); put(D, 4)
    put(Bq, 4); put(A, 1, a_slots); put(D, 4); put(C, 1); put(Bq, 1); put(D, 1)
    bm.free_seq(D)
    assert bm.table(A) == gold["tables"]["A"]
    assert bm.table(Bq) == gold["tables"]["B"]
    assert bm.table(C) == gold["tables"]["C"]
    assert sorted(bm.free) == gold["free_pages"]
    assert a_slots == gold["A_slots"]
    assert len(gold["request_A_tokens"]) - B * (len(bm.table(A)) - 1) == gold["A_tokens_in_last_block"]
    bm.check_invariants()

    # De-paging A's pool returns its 9 tokens in logical order; free pages stay untouched (NaN).
    H, Dm = 1, 16
    kp = host_pool(12, H, Dm, "f32", B=B, fill=np.nan)
    vp = host_pool(12, H, Dm, "f32", B=B, fill=np.nan)
    tok = np.arange(9, dtype=np.float32)[:, None] * np.ones((1, Dm), np.float32)
    oracle.reshape_and_cache(kp, vp, "f32", None, None, 12, H, Dm, tok, -tok, "f32",
                             np.array(a_slots), B=B)
    kc, vc = oracle.gather(kp, vp, "f32", None, None, 12, H, Dm, np.array(gold["tables"]["A"]), 9,
                           0, B=B)
    assert np.array_equal(kc, tok.astype(np.float64)) and np.array_equal(vc, -tok.astype(np.float64))
    for page in gold["free_pages"] + gold["tables"]["B"] + gold["tables"]["C"]:
        span = slice(page * B * Dm, (page + 1) * B * Dm)
        assert np.all(np.isnan(kp[span])) and np.all(np.isnan(vp[span]))


# ------------------------------------------------------------------------ reshape + gather round trip
def _values(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g)
    return x.to({"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype])


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_reshape_then_gather_returns_the_rows(dtype):
    H, D, nb, B = 2, 64, 24, 16
    L = 37
    perm = np.random.default_rng(1).permutation(nb)[: -(-L // B)].astype(np.int32)
    slots = np.array([perm[p // B] * B + p % B for p in range(L)], np.int64)
    k = _values((L, H, D), dtype, 3)
    v = _values((L, H, D), dtype, 4)
    kp = host_pool(nb, H, D, dtype)
    vp = host_pool(nb, H, D, dtype)
    oracle.reshape_and_cache(kp, vp, dtype, None, None, nb, H, D, raw(k), raw(v), dtype, slots)
    for h in range(H):
        kc, vc = oracle.gather(kp, vp, dtype, None, None, nb, H, D, perm, L, h)
        assert np.array_equal(kc, k[:, h].double().numpy())
        assert np.array_equal(vc, v[:, h].double().numpy())


def test_reshape_fp8_matches_torch_quantisation():
    H, D, nb, B = 2, 64, 8, 16
    L = 20
    table = np.array([5, 2], np.int32)
    slots = np.array([table[p // B] * B + p % B for p in range(L)], np.int64)
    k = _values((L, H, D), "f16", 5) * 3
    v = _values((L, H, D), "f16", 6)
    ks = np.array([0.05, 0.04], np.float32)   # |k| <= ~15 here, so |k / s| stays below 448
    vs = np.array([0.01, 0.03], np.float32)
    kp = host_pool(nb, H, D, "fp8")
    vp = host_pool(nb, H, D, "fp8")
    oracle.reshape_and_cache(kp, vp, "fp8", ks, vs, nb, H, D, raw(k), raw(v), "f16", slots)
    for h in range(H):
        kc, vc = oracle.gather(kp, vp, "fp8", ks, vs, nb, H, D, table, L, h)
        # torch: binary32 division, then float8_e4m3fn rounding, then back (values stay < 448 here)
        kq = (k[:, h].float() / torch.tensor(ks[h])).to(torch.float8_e4m3fn).double() * float(ks[h])
        vq = (v[:, h].float() / torch.tensor(vs[h])).to(torch.float8_e4m3fn).double() * float(vs[h])
        assert np.array_equal(kc, kq.numpy()) and np.array_equal(vc, vq.numpy())


def test_reshape_skips_negative_and_out_of_range_slots():
    H, D, nb = 1, 64, 2
    kp = host_pool(nb, H, D, "f32", fill=7.0)
    vp = host_pool(nb, H, D, "f32", fill=7.0)
    rows = np.ones((3, H * D), np.float32)
    oracle.reshape_and_cache(kp, vp, "f32", None, None, nb, H, D, rows, rows, "f32",
                             np.array([-1, nb * 16, nb * 16 + 5]))
    assert np.all(kp == 7.0) and np.all(vp == 7.0)


# ------------------------------------------------------------------------ attention
def _sdpa(q, k, v, scale):
    """torch scaled_dot_product_attention in float64 on contiguous rows: q [D], k/v [L][D]."""
    qt = torch.as_tensor(q, dtype=torch.float64)[None, None, None, :]
    kt = torch.as_tensor(k, dtype=torch.float64)[None, None]
    vt = torch.as_tensor(v, dtype=torch.float64)[None, None]
    return F.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, 0, 0].numpy()


@pytest.mark.parametrize("L", [1, 2, 17, 100])
def test_attend_matches_torch_sdpa(L):
    g = np.random.default_rng(L)
    D = 64
    q, k, v = g.standard_normal(D), g.standard_normal((L, D)), g.standard_normal((L, D))
    out = oracle.attend_contiguous(q, k, v, 0.125)
    assert np.max(np.abs(out - _sdpa(q, k, v, 0.125))) < 1e-12


def _paged_problem(dtype, lengths, Hq, H, D, nb, seed, perm_seed=11):
    """Random logical K/V per sequence written into a host pool through the oracle's replay, with
    physical blocks taken from a seeded permutation."""
    B = 16
    S = len(lengths)
    M = max(-(-int(L) // B) for L in lengths)
    perm = list(np.random.default_rng(perm_seed).permutation(nb))
    tables = np.full((S, M), -7, np.int32)
    kp = host_pool(nb, H, D, dtype, fill=nan_bits(dtype))
    vp = host_pool(nb, H, D, dtype, fill=nan_bits(dtype))
    logical = []
    for s, L in enumerate(lengths):
        nblk = -(-int(L) // B)
        for j in range(nblk):
            tables[s, j] = perm.pop()
        k = _values((int(L), H, D), dtype, seed + 2 * s)
        v = _values((int(L), H, D), dtype, seed + 2 * s + 1)
        slots = np.array([tables[s, p // B] * B + p % B for p in range(int(L))], np.int64)
        oracle.reshape_and_cache(kp, vp, dtype, None, None, nb, H, D, raw(k), raw(v), dtype, slots)
        logical.append((k, v))
    q = _values((S, Hq, D), dtype, seed + 999)
    return q, kp, vp, tables, logical


def test_decode_matches_sdpa_with_gqa_and_scattered_blocks():
    lengths = [5, 16, 17, 40]
    Hq, H, D, nb = 4, 2, 64, 32
    q, kp, vp, tables, logical = _paged_problem("f32", lengths, Hq, H, D, nb, 100)
    out = oracle.decode_attention(raw(q), "f32", kp, vp, "f32", None, None, nb, H, D, tables,
                                  np.array(lengths), Hq, 0.125)
    for s, (k, v) in enumerate(logical):
        # grouped heads: query head hq reads KV head hq // (Hq // H)
        kk = k.double().repeat_interleave(Hq // H, dim=1)
        vv = v.double().repeat_interleave(Hq // H, dim=1)
        for hq in range(Hq):
            ref = _sdpa(q[s, hq].double().numpy(), kk[:, hq].numpy(), vv[:, hq].numpy(), 0.125)
            assert np.max(np.abs(out[s, hq] - ref)) < 1e-12


def test_decode_fp8_cache_matches_sdpa_on_dequantised_values():
    H, Hq, D, nb, B = 2, 4, 64, 16, 16
    L = 33
    table = np.array([[9, 3, 12]], np.int32)
    slots = np.array([table[0, p // B] * B + p % B for p in range(L)], np.int64)
    k = _values((L, H, D), "f16", 21)
    v = _values((L, H, D), "f16", 22)
    ks = np.array([4.0 / 448, 3.5 / 448], np.float32)
    vs = np.array([4.2 / 448, 3.9 / 448], np.float32)
    kp = host_pool(nb, H, D, "fp8")
    vp = host_pool(nb, H, D, "fp8")
    oracle.reshape_and_cache(kp, vp, "fp8", ks, vs, nb, H, D, raw(k), raw(v), "f16", slots)
    q = _values((1, Hq, D), "f16", 23)
    out = oracle.decode_attention(raw(q), "f16", kp, vp, "fp8", ks, vs, nb, H, D, table,
                                  np.array([L]), Hq, 0.125)
    for hq in range(Hq):
        h = hq // 2
        kq = (k[:, h].float() / float(ks[h])).to(torch.float8_e4m3fn).double() * float(ks[h])
        vq = (v[:, h].float() / float(vs[h])).to(torch.float8_e4m3fn).double() * float(vs[h])
        ref = _sdpa(q[0, hq].double().numpy(), kq.numpy(), vq.numpy(), 0.125)
        assert np.max(np.abs(out[0, hq] - ref)) < 1e-12


def _single_seq(k, v, q, Hq=2, H=1, D=64, nb=8, table=(6, 1, 4, 0)):
    L = k.shape[0]
    t = np.array([list(table)[: -(-L // 16)]], np.int32)
    slots = np.array([t[0, p // 16] * 16 + p % 16 for p in range(L)], np.int64)
    kp = host_pool(nb, H, D, "f32", fill=np.nan)
    vp = host_pool(nb, H, D, "f32", fill=np.nan)
    oracle.reshape_and_cache(kp, vp, "f32", None, None, nb, H, D,
                             np.ascontiguousarray(k, np.float32), np.ascontiguousarray(v, np.float32),
                             "f32", slots)
    return oracle.decode_attention(np.ascontiguousarray(q, np.float32), "f32", kp, vp, "f32", None,
                                   None, nb, H, D, t, np.array([L]), Hq, 0.125)[0]


def test_closed_forms():
    g = np.random.default_rng(5)
    D = 64
    # L = 1: the only value row comes back exactly.
    k, v = g.standard_normal((1, D)), g.standard_normal((1, D))
    q = g.standard_normal((1, 2 * D))
    out = _single_seq(k, v, q)
    assert np.array_equal(out[0], v[0].astype(np.float32).astype(np.float64))
    # q = 0: every weight is equal -> the mean of the value rows (here over 3 blocks).
    L = 40
    k, v = g.standard_normal((L, D)), g.standard_normal((L, D))
    out = _single_seq(k, v, np.zeros((1, 2 * D)))
    mean = v.astype(np.float32).astype(np.float64).mean(axis=0)
    assert np.max(np.abs(out[0] - mean)) < 1e-12
    # constant value rows -> that row, whatever the scores.
    row = g.standard_normal(D)
    out = _single_seq(k, np.tile(row, (L, 1)), g.standard_normal((1, 2 * D)))
    assert np.max(np.abs(out - row.astype(np.float32))) < 1e-12
    # two tokens: weights are the logistic function of the score difference.
    a = 3.0
    q = np.zeros((1, 2 * D)); q[0, 0] = a; q[0, D] = -a
    k = np.zeros((2, D)); k[0, 0] = 1.0
    v = g.standard_normal((2, D)).astype(np.float32)
    out = _single_seq(k, v, q)
    sig = 1.0 / (1.0 + math.exp(-a * 0.125))
    v64 = v.astype(np.float64)
    assert np.max(np.abs(out[0] - (sig * v64[0] + (1 - sig) * v64[1]))) < 1e-12
    assert np.max(np.abs(out[1] - ((1 - sig) * v64[0] + sig * v64[1]))) < 1e-12
    # one key aligned with the query at a huge score: its value row wins (max subtraction keeps
    # the exponentials finite).
    k = g.standard_normal((L, D)) * 0.01
    q = np.zeros((1, 2 * D)); q[0, 3] = 1000.0; q[0, D + 3] = 1000.0
    k[29, 3] = 100.0
    v = g.standard_normal((L, D)).astype(np.float32)
    out = _single_seq(k, v=v, q=q)
    assert np.array_equal(out[0], v[29].astype(np.float64))
    assert np.array_equal(out[1], v[29].astype(np.float64))


def test_gqa_head_mapping():
    # Each KV head carries constant value rows equal to its index: query head hq must return
    # hq // group in every component.
    Hq, H, D, nb = 8, 4, 64, 8
    L = 21
    table = np.array([[3, 6]], np.int32)
    slots = np.array([table[0, p // 16] * 16 + p % 16 for p in range(L)], np.int64)
    g = np.random.default_rng(9)
    k = g.standard_normal((L, H, D)).astype(np.float32)
    v = np.broadcast_to(np.arange(H, dtype=np.float32)[None, :, None], (L, H, D)).copy()
    kp = host_pool(nb, H, D, "f32", fill=np.nan)
    vp = host_pool(nb, H, D, "f32", fill=np.nan)
    oracle.reshape_and_cache(kp, vp, "f32", None, None, nb, H, D, k, v, "f32", slots)
    q = g.standard_normal((1, Hq * D)).astype(np.float32)
    out = oracle.decode_attention(q, "f32", kp, vp, "f32", None, None, nb, H, D, table,
                                  np.array([L]), Hq, 0.125)
    for hq in range(Hq):
        assert np.allclose(out[0, hq], hq // 2, atol=1e-12)


def test_permutation_of_physical_blocks_changes_nothing():
    lengths = [5, 16, 17, 40]
    outs = []
    for perm_seed in (11, 12, 13):
        q, kp, vp, tables, _ = _paged_problem("f16", lengths, 4, 2, 64, 32, 200, perm_seed)
        outs.append(oracle.decode_attention(raw(q), "f16", kp, vp, "f16", None, None, 32, 2, 64,
                                            tables, np.array(lengths), 4, 0.125))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_shared_prefix_equals_duplicated_prefix():
    H, Hq, D, nb, B = 2, 4, 64, 64, 16
    pre, suf = 32, [3, 20, 9]
    g = torch.Generator().manual_seed(31)
    kpre = torch.randn((pre, H, D), generator=g).half()
    vpre = torch.randn((pre, H, D), generator=g).half()
    q = torch.randn((len(suf), Hq, D), generator=g).half()
    sufkv = [(torch.randn((n, H, D), generator=g).half(), torch.randn((n, H, D), generator=g).half())
             for n in suf]
    lengths = np.array([pre + n for n in suf], np.int32)
    M = -(-int(lengths.max()) // B)
    results = []
    for shared in (True, False):
        kp = host_pool(nb, H, D, "f16", fill=nan_bits("f16"))
        vp = host_pool(nb, H, D, "f16", fill=nan_bits("f16"))
        free = list(range(nb))[::-1]
        tables = np.full((len(suf), M), -1, np.int32)
        prefix_blocks = [free.pop() for _ in range(pre // B)]
        for s, n in enumerate(suf):
            blocks = prefix_blocks if shared else [free.pop() for _ in range(pre // B)]
            blocks = blocks + [free.pop() for _ in range(-(-n // B))]
            tables[s, : len(blocks)] = blocks
            kk = torch.cat([kpre, sufkv[s][0]])
            vv = torch.cat([vpre, sufkv[s][1]])
            L = pre + n
            slots = np.array([tables[s, p // B] * B + p % B for p in range(L)], np.int64)
            oracle.reshape_and_cache(kp, vp, "f16", None, None, nb, H, D, raw(kk), raw(vv), "f16",
                                     slots)
        results.append(oracle.decode_attention(raw(q), "f16", kp, vp, "f16", None, None, nb, H, D,
                                               tables, lengths, Hq, 0.125))
    assert np.array_equal(results[0], results[1])


def test_nan_poison_outside_the_context_is_never_read():
    lengths = [5, 16, 17, 40]
    q, kp, vp, tables, _ = _paged_problem("bf16", lengths, 4, 2, 64, 32, 300)
    out = oracle.decode_attention(raw(q), "bf16", kp, vp, "bf16", None, None, 32, 2, 64, tables,
                                  np.array(lengths), 4, 0.125)
    assert np.all(np.isfinite(out))  # unused blocks, tail slots and padding are all NaN/-7 here


def test_zero_length_gives_zero_and_bad_block_id_is_rejected():
    q, kp, vp, tables, _ = _paged_problem("f32", [0, 7], 4, 2, 64, 8, 400)
    tables[0, :] = -7
    out = oracle.decode_attention(raw(q), "f32", kp, vp, "f32", None, None, 8, 2, 64, tables,
                                  np.array([0, 7]), 4, 0.125)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    tables[1, 0] = 8  # one past the pool
    with pytest.raises(ValueError):
        oracle.decode_attention(raw(q), "f32", kp, vp, "f32", None, None, 8, 2, 64, tables,
                                np.array([0, 7]), 4, 0.125)


def test_selected_pairs_match_the_full_result():
    lengths = [5, 16, 17, 40]
    q, kp, vp, tables, _ = _paged_problem("f16", lengths, 4, 2, 64, 32, 500)
    full = oracle.decode_attention(raw(q), "f16", kp, vp, "f16", None, None, 32, 2, 64, tables,
                                   np.array(lengths), 4, 0.125)
    ss = np.array([3, 0, 2, 3]); hh = np.array([1, 3, 0, 2])
    part = oracle.decode_attention(raw(q), "f16", kp, vp, "f16", None, None, 32, 2, 64, tables,
                                   np.array(lengths), 4, 0.125, sel=(ss, hh))
    assert np.array_equal(part, full[ss, hh])


# ------------------------------------------------------------------------ copy-on-write replay
def test_copy_blocks_clone_then_write_leaves_the_sharer_untouched():
    # Two sequences share one partially filled block; the writer gets a clone and writes its next
    # token there: afterwards the writer sees old tokens + the new one, the sharer only the old.
    H, D, nb, B = 1, 64, 6, 16
    kp = host_pool(nb, H, D, "f16", fill=nan_bits("f16"))
    vp = host_pool(nb, H, D, "f16", fill=nan_bits("f16"))
    old_k = _values((10, H, D), "f16", 41)
    old_v = _values((10, H, D), "f16", 42)
    oracle.reshape_and_cache(kp, vp, "f16", None, None, nb, H, D, raw(old_k), raw(old_v), "f16",
                             np.arange(2 * B, 2 * B + 10))
    oracle.copy_blocks([kp], [vp], H * B * D * 2, nb, np.array([[2, 5]]))
    new_k = _values((1, H, D), "f16", 43)
    new_v = _values((1, H, D), "f16", 44)
    oracle.reshape_and_cache(kp, vp, "f16", None, None, nb, H, D, raw(new_k), raw(new_v), "f16",
                             np.array([5 * B + 10]))
    kw, vw = oracle.gather(kp, vp, "f16", None, None, nb, H, D, np.array([5]), 11, 0)
    ko, vo = oracle.gather(kp, vp, "f16", None, None, nb, H, D, np.array([2]), 10, 0)
    assert np.array_equal(kw[:10], old_k[:, 0].double().numpy())
    assert np.array_equal(kw[10], new_k[0, 0].double().numpy())
    assert np.array_equal(vw[10], new_v[0, 0].double().numpy())
    assert np.array_equal(ko, old_k[:, 0].double().numpy())
    assert np.array_equal(vo, old_v[:, 0].double().numpy())
    assert np.all(np.isnan(oracle.gather(kp, vp, "f16", None, None, nb, H, D, np.array([2]), 11,
                                         0)[0][10].astype(np.float64)))


def test_copy_blocks_skips_out_of_range_pairs_and_touches_nothing_else():
    H, D, nb = 2, 64, 4
    g = np.random.default_rng(3)
    kp = g.standard_normal(nb * H * 16 * D).astype(np.float32)
    vp = g.standard_normal(nb * H * 16 * D).astype(np.float32)
    k0, v0 = kp.copy(), vp.copy()
    oracle.copy_blocks([kp], [vp], H * 16 * D * 4, nb, np.array([[0, 3], [1, 4], [-1, 2]]))
    blk = H * 16 * D
    assert np.array_equal(kp[3 * blk:], k0[:blk]) and np.array_equal(vp[3 * blk:], v0[:blk])
    assert np.array_equal(kp[: 3 * blk], k0[: 3 * blk]) and np.array_equal(vp[: 3 * blk], v0[: 3 * blk])


def test_swap_replay_copies_whole_blocks_both_ways():
    """Swapping: a block's bytes go to its host slot and come back unchanged; other bytes of either
    pool are untouched; pairs outside a pool are skipped."""
    g = np.random.default_rng(7)
    bb, nb, nh = 24, 6, 3
    dev = [g.integers(0, 256, nb * bb).astype(np.uint8) for _ in range(4)]  # 2 layers x K, V
    host = [np.zeros(nh * bb, np.uint8) for _ in range(4)]
    orig = [x.copy() for x in dev]
    oracle.swap_blocks(dev, host, bb, nb, nh, [(4, 2), (0, 0), (nb, 1), (1, nh)], True)
    for x, hx in zip(orig, host):
        assert np.array_equal(hx[2 * bb:3 * bb], x[4 * bb:5 * bb])
        assert np.array_equal(hx[0:bb], x[0:bb])
        assert not hx[bb:2 * bb].any()  # slot 1: its pair named a block outside the pool
    for x in dev:
        x[:] = 0
    oracle.swap_blocks(dev, host, bb, nb, nh, [(5, 2), (3, 0)], False)
    for x, o in zip(dev, orig):
        assert np.array_equal(x[5 * bb:6 * bb], o[4 * bb:5 * bb])
        assert np.array_equal(x[3 * bb:4 * bb], o[0:bb])
        assert not x[:3 * bb].any() and not x[4 * bb:5 * bb].any()


# ------------------------------------------------------------------------ prefill (a chunk per sequence)
def test_prefill_matches_causal_sdpa_on_contiguous_kv():
    """A chunk of new tokens per sequence against torch's scaled_dot_product_attention with its own
    causal mask (is_causal) on the de-paged K/V: the last n_s query rows of an L_s x L_s causal
    attention."""
    lengths = [7, 16, 40, 3]
    chunks = [7, 5, 17, 0]  # whole prompt, a chunk ending mid-block, a long chunk, nothing
    Hq, H, D, nb = 4, 2, 64, 24
    _, kp, vp, tables, logical = _paged_problem("f32", lengths, Hq, H, D, nb, 500)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = _values((int(qs[-1]), Hq, D), "f32", 501)
    out = oracle.prefill_attention(raw(q).reshape(int(qs[-1]), -1), "f32", kp, vp, "f32", None,
                                   None, nb, H, D, tables, np.array(lengths), qs, Hq, 0.125)
    for s, ((k, v), L, n) in enumerate(zip(logical, lengths, chunks)):
        if n == 0:
            continue
        kk = k.double().repeat_interleave(Hq // H, dim=1).permute(1, 0, 2)  # [Hq, L, D]
        vv = v.double().repeat_interleave(Hq // H, dim=1).permute(1, 0, 2)
        # queries for all L positions; only the last n are the chunk's
        qq = torch.zeros(Hq, L, D, dtype=torch.float64)
        qq[:, L - n:] = q[qs[s]:qs[s + 1]].double().permute(1, 0, 2)
        ref = F.scaled_dot_product_attention(qq[None], kk[None], vv[None], is_causal=True,
                                             scale=0.125)[0]
        got = torch.from_numpy(out[qs[s]:qs[s + 1]]).permute(1, 0, 2)
        assert torch.max(torch.abs(got - ref[:, L - n:])) < 1e-12


def test_prefill_closed_forms():
    """The first token of a prompt sees only itself: its output is its own V row.  With every key
    equal, token p's output is the mean of V[0..p]."""
    L, Hq, H, D, nb = 20, 2, 1, 64, 8
    _, kp, vp, tables, logical = _paged_problem("f32", [L], Hq, H, D, nb, 600)
    qs = np.array([0, L], np.int32)
    q = _values((L, Hq, D), "f32", 601)
    out = oracle.prefill_attention(raw(q).reshape(L, -1), "f32", kp, vp, "f32", None, None, nb, H,
                                   D, tables, np.array([L]), qs, Hq, 0.125)
    v = logical[0][1].double().numpy()  # [L, H, D]
    assert np.max(np.abs(out[0, :, :] - v[0, 0])) < 1e-12
    # equal keys: rewrite every K row of the pool to one vector, then token p averages V[0..p]
    k_all = np.tile(raw(logical[0][0][:1]), (L, 1, 1))
    slots = np.array([tables[0, p // 16] * 16 + p % 16 for p in range(L)], np.int64)
    oracle.reshape_and_cache(kp, vp, "f32", None, None, nb, H, D, k_all, raw(logical[0][1]), "f32",
                             slots)
    out = oracle.prefill_attention(raw(q).reshape(L, -1), "f32", kp, vp, "f32", None, None, nb, H,
                                   D, tables, np.array([L]), qs, Hq, 0.125)
    for p in range(L):
        assert np.max(np.abs(out[p, :, :] - v[: p + 1, 0].mean(axis=0))) < 1e-12


# ------------------------------------------------------------------------ block size
@pytest.mark.parametrize("dtype", ["f16", "fp8"])
def test_block_size_changes_the_layout_not_the_result(dtype):
    """The block size only decides where positions land ("PagedAttention" (devoured.fyi), "Why the
    attention kernel works at all": the math is untouched by the layout): the same sequences
    written into pools of 8-, 16- and 32-position blocks, through tables from a block manager of
    that size, give bitwise the same oracle output, which matches SDPA on the rows."""
    from oracle.bm_model import BlockManagerModel
    H, Hq, D = 2, 6, 64
    lengths = [5, 16, 17, 40, 33, 8]
    kd = "f16"
    k = [_values((L, H, D), kd, 40 + i) for i, L in enumerate(lengths)]
    v = [_values((L, H, D), kd, 60 + i) for i, L in enumerate(lengths)]
    q = _values((len(lengths), Hq, D), kd, 80)
    ks = vs = None
    if dtype == "fp8":  # amax / 448 per head: every value is inside the E4M3 range
        ks = (torch.cat(k).float().abs().amax(dim=(0, 2)) / 448).numpy().astype(np.float32)
        vs = (torch.cat(v).float().abs().amax(dim=(0, 2)) / 448).numpy().astype(np.float32)
    outs = {}
    for B in (8, 16, 32):
        nb = 256 // B
        bm = BlockManagerModel(nb, B, np.random.default_rng(B).permutation(nb))
        seqs = [bm.add_seq() for _ in lengths]
        slots = [[bm.append(s)[0] for _ in range(L)] for s, L in zip(seqs, lengths)]
        M = max(-(-L // B) for L in lengths)
        rows, ctx = bm.export(seqs, M, 0)
        kp = host_pool(nb, H, D, dtype, B=B, fill=nan_bits(dtype))
        vp = host_pool(nb, H, D, dtype, B=B, fill=nan_bits(dtype))
        oracle.reshape_and_cache(kp, vp, dtype, ks, vs, nb, H, D, raw(torch.cat(k)), raw(torch.cat(v)),
                                 kd, np.concatenate(slots).astype(np.int64), B=B)
        outs[B] = oracle.decode_attention(raw(q).reshape(len(lengths), -1), kd, kp, vp, dtype, ks,
                                          vs, nb, H, D, np.array(rows, np.int32),
                                          np.array(ctx, np.int32), Hq, 0.125, B=B)
    assert np.array_equal(outs[8], outs[16]) and np.array_equal(outs[32], outs[16])
    for s, L in enumerate(lengths):
        for hq in range(Hq):
            h = hq // (Hq // H)
            kk, vv = k[s][:, h].double(), v[s][:, h].double()
            if dtype == "fp8":
                kk = (k[s][:, h].float() / float(ks[h])).to(torch.float8_e4m3fn).double() * float(ks[h])
                vv = (v[s][:, h].float() / float(vs[h])).to(torch.float8_e4m3fn).double() * float(vs[h])
            ref = _sdpa(q[s, hq].double().numpy(), kk.numpy(), vv.numpy(), 0.125)
            assert np.max(np.abs(outs[16][s, hq] - ref)) < 1e-12


def test_layout_indices_of_an_8_position_block():
    """Worked by hand from the layout description with B = 8 (H = 2 KV heads, D = 64, f16 so 8
    elements per 16-byte vector): K element (t, i) of tile (b, h) sits at
    (b*H + h)*B*D + ((i // 8)*B + t)*8 + i % 8; V element (t, i) at (b*H + h)*B*D + i*B + t."""
    H, D, B = 2, 64, 8
    # block 3, head 1, position 5, dim 19: tile 7*512 = 3584; K ((2*8 + 5)*8 + 3) = 171; V 19*8 + 5
    assert oracle.k_index(3, 1, 5, 19, H, D, B, "f16") == 3584 + 171
    assert oracle.v_index(3, 1, 5, 19, H, D, B) == 3584 + 157
    # block 0, head 0, position 7, dim 63: K (7*8 + 7)*8 + 7 = 511 (the tile's last element)
    assert oracle.k_index(0, 0, 7, 63, H, D, B, "f16") == 511


def test_oracle_refuses_pools_smaller_than_their_geometry():
    """A pool of 8-position blocks read as 16-position blocks would be indexed past its end: the
    oracle's wrappers refuse it before the C routines run."""
    nb, H, D = 4, 1, 8
    kp = np.zeros(oracle.pool_elems(nb, H, D, 8), np.float32)
    vp = np.zeros_like(kp)
    q = np.zeros((1, D), np.float32)
    table = np.array([[3, 2, 1, 0]], np.int32)
    ctx = np.array([20], np.int32)
    oracle.decode_attention(q, "f32", kp, vp, "f32", None, None, nb, H, D, table, ctx, 1, 1.0, B=8)
    with pytest.raises(ValueError, match="fewer than"):
        oracle.decode_attention(q, "f32", kp, vp, "f32", None, None, nb, H, D, table, ctx, 1, 1.0)
    with pytest.raises(ValueError, match="fewer than"):
        oracle.gather(kp, vp, "f32", None, None, nb, H, D, table[0], 20, 0)
