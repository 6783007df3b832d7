#!/usr/bin/env python3
"""Benchmark of decode-step paged attention on one MI355X.

A step is one pass of the whole hot path over one batch: the copy-on-write clone (when the step has
pairs), then for every layer reshape_and_cache of the new token and the split-K decode with its
partition reduce.  The step's metadata (slots, tables, lengths, copy pairs) comes from the host
block manager before timing and is resident in HBM when the timed region starts.

Prints ONE JSON line (default workload: the shared-prefix batch of 256 sequences):
  value        KV GB/s of the step: algorithmic KV bytes read per step / step time, the median of
               several passes of the timed loop (unique physical slots for the shared-prefix
               workload, whose logical bytes count the prefix once per sequence; logical otherwise);
  roofline     for pa_decode_attention (the dominant call: split-K kernel + partition reduce):
               algorithmic bytes per call (unique physical KV slots + tables + lengths + Q + out)
               / its mean duration from HIP events on the launch stream, against 8 TB/s;
  cpu_baseline the CPU oracle (fp64) timed on the host's cores on a bounded sample of set 0, and on
               one core;
  calibration  the read-bandwidth reference (pa_calibrate_read): a plain read of exactly the tiles
               a decode call reads, and a sequential read of 2 GiB, on the same device;
  targets      the 32K-context bf16 batch's decode call measured in the same run (default run);
  decode_call_us, reshape_call_us, copy_call_us
               p10 / p50 / p90 / mean per call over 20 batches of back-to-back eager calls,
               and seqs_per_s_per_layer_calls = S / (decode + reshape + copy / layers), medians.

Timing loops rotate between `--sets` independent batches of the workload placed in the same pool
(distinct blocks and values), so each step reads KV that the 256 MB MALL and the L2s do not already
hold, as the successive layers of a model would.  Calls are launched from Python, which stays ahead
of the GPU on every workload here (--graph replays each set's step as a captured HIP graph instead);
the decode-call duration is the mean of back-to-back decode calls between two HIP events on the
stream they run on.
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "paged decode attention KV GB/s (% of HBM peak) + sequences/s per layer"
# independent batches rotated by the timing loop, so that successive steps read KV that no cache
# holds (the 256 MB MALL included); the 28-layer step reads ~14.5 GB by itself
DEFAULT_WORKLOAD = "f16_shared_prefix_batch256"
DEFAULT_SETS = {"tiny_f32": 1, "f16_batch32": 16, "bf16_32k_batch8": 3,
                "f16_shared_prefix_batch256": 4, "fp8_28layer_batch512": 1}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(batch, unique: bool) -> int:
    """Bytes one pa_decode_attention call must move at minimum: the KV rows of every context
    position (each distinct physical slot once when unique), the block-table entries and lengths
    it reads, the queries it reads and the outputs it writes (fp8: plus the per-head scales)."""
    w = batch.w
    kv = batch.kv_bytes_per_layer(unique=unique)
    tables = int(sum(math.ceil(int(L) / w.block_size) for L in batch.lengths)) * 4
    lens = w.num_seqs * 4
    qe = 4 if w.q_dtype == "f32" else 2
    qo = 2 * w.num_seqs * w.num_q_heads * w.head_dim * qe
    sc = 2 * w.num_kv_heads * 4 if w.cache_dtype == "fp8" else 0
    return kv + tables + lens + qo + sc


def tile_list(batch, r: int) -> np.ndarray:
    """Tile indices (block * num_kv_heads + head) that a decode call of set r reads: every
    sequence's blocks up to its context length, for every KV head, each distinct tile once (a shared
    prefix's blocks count once), in (sequence, block, head) order."""
    w = batch.w
    st = batch.sets[r]
    B, H = w.block_size, w.num_kv_heads
    seen, out = set(), []
    for s in range(w.num_seqs):
        for j in range(-(-int(st.ctx[s]) // B)):
            b = int(st.tables[s, j])
            if b in seen or not 0 <= b < w.num_blocks:
                continue
            seen.add(b)
            out.extend(b * H + h for h in range(H))
    return np.asarray(out, np.int32)


def calibration(batch, torch, api, sets: int) -> dict:
    """pa_calibrate_read on this device: the tiles the decode reads (rotating over the sets and
    layers as the decode timing does, so no cache holds them), and a sequential read of up to 1 GiB
    per pool."""
    w = batch.w
    e = 1 if w.cache_dtype == "fp8" else (4 if w.cache_dtype == "f32" else 2)
    tb = w.block_size * w.head_dim * e
    if tb % 1024:
        return None
    lists = [torch.from_numpy(tile_list(batch, r)).cuda() for r in range(sets)]
    lay = list(batch.layers)
    n_seq0 = min(batch.caches[lay[0]].k_pool.numel(), 1 << 30) // tb
    sink = torch.empty((max(n_seq0, max(t.numel() for t in lists)) + 3) // 4, dtype=torch.int32,
                       device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn, n, reps=10):
        for k in range(n):
            fn(k)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for k in range(n * reps):
            fn(k)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1e3 / (n * reps)

    def gather(k):
        c = batch.caches[lay[(k // sets) % len(lay)]]
        t = lists[k % sets]
        api.pa_calibrate_read(c.k_pool, c.v_pool, tb, t, t.numel(), sink)

    n = max(4, sets * len(lay))
    sec_g = timed(gather, n)
    g_bytes = 2 * lists[0].numel() * tb
    c0 = batch.caches[lay[0]]
    n_seq = min(c0.k_pool.numel(), 1 << 30) // tb
    sec_s = timed(lambda k: api.pa_calibrate_read(c0.k_pool, c0.v_pool, tb, None, n_seq, sink), 2)
    s_bytes = 2 * n_seq * tb
    return {"kernel": "pa_calibrate_read", "waves": "one per tile",
            "gather_GBps": round(g_bytes / sec_g / 1e9, 1), "gather_bytes": g_bytes,
            "gather_us": round(sec_g * 1e6, 2),
            "sequential_GBps": round(s_bytes / sec_s / 1e9, 1), "sequential_bytes": s_bytes,
            "note": "plain reads of the decode call's own tiles (each distinct tile once) and of a "
                    "contiguous range; the achievable rate on this device for those bytes"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_traffic(w, default_run: bool, partition_size: int):
    """HBM bytes per decode call from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs summarised in
    profiles/traffic.json (scaled by the reference copy), or None when this run is not the measured
    configuration (the same workload and call partition size) or the kernel sources have changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not default_run or not os.path.exists(path):
        return None
    t = json.load(open(path))
    h = hashlib.sha256()
    for f in t["kernel_sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != t["sha256"] or w.name not in t["workloads"]:
        return None
    rec = t["workloads"][w.name]
    if rec.get("partition_size") != partition_size:
        return None
    return int(rec["bytes_per_call"])


def cpu_baseline(batch, budget_s: float) -> dict:
    """The CPU oracle, as it stands, on a bounded sample of set 0 of layer 0: whole sequences (all
    query heads) taken in order until the estimated work fits the budget; repeated until the
    measured time reaches the budget (ten seconds by default)."""
    import oracle
    from oracle.batch import OracleBatch

    w = batch.w
    L = batch.lengths.astype(np.int64)
    # estimate: ~4 ns per (position, head-dim, query head) on one core for de-page + dot products,
    # plus rebuilding the sequence's history in the oracle's pool first (one thread): ~1.2 us per
    # element for the fp8 encoder (an exact search over the codes), ~5 ns for bit copies
    threads = oracle.max_threads()
    enc = 1.2e-6 if w.cache_dtype == "fp8" else 5e-9
    per_seq = L * w.num_q_heads * w.head_dim * 4e-9 * 2 / max(threads, 1) + \
        L * 2 * w.num_kv_heads * w.head_dim * enc
    take, acc = [], 0.0
    for s in range(w.num_seqs):
        if take and acc + per_seq[s] > budget_s:
            break
        take.append(s)
        acc += per_seq[s]
    layer = batch.layers[0]
    ob = OracleBatch(batch, pad_block=0)
    ob.metadata_matches(batch)
    ob.build_pools(batch, layer, owners=set(take))
    sel = (np.repeat(take, w.num_q_heads), np.tile(np.arange(w.num_q_heads), len(take)))
    e = 1 if w.cache_dtype == "fp8" else (4 if w.cache_dtype == "f32" else 2)
    row = 2 * w.num_kv_heads * w.head_dim * e
    # per query head the oracle de-pages its KV head's rows: count the logical bytes of the sample
    sample_bytes = int(L[take].sum()) * row
    def run(nthreads, budget, sel):
        t0 = time.perf_counter()
        reps = 0
        while True:
            ob.attention(batch, layer, sel=sel, nthreads=nthreads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 1000:
                return reps, el

    reps, el = run(threads, budget_s, sel)
    gbps = sample_bytes * reps / el / 1e9
    # one core: the first sequences of the same sample, bounded to a fifth of the budget
    frac = (budget_s / 5) / max(acc * max(threads, 1), 1e-9)
    one = take[:max(1, min(len(take), int(len(take) * frac)))]
    sel1 = (np.repeat(one, w.num_q_heads), np.tile(np.arange(w.num_q_heads), len(one)))
    reps1, el1 = run(1, budget_s / 5, sel1)
    bytes1 = int(L[one].sum()) * row
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"layer {layer}, set 0: {len(take)} of {w.num_seqs} sequences x all "
                      f"{w.num_q_heads} query heads ({int(L[take].sum())} positions), fp64, "
                      f"{reps} pass(es) in {el:.2f} s; seqs/s = "
                      f"{len(take) * reps / el:.3f}",
            "one_core": {"value": round(bytes1 * reps1 / el1 / 1e9, 4), "unit": "GB/s",
                         "sample": f"{len(one)} sequence(s) of the same sample, {reps1} pass(es) "
                                   f"in {el1:.2f} s on 1 thread"}}


def swap_bench(args, torch, api, wl, DecodeBatch) -> int:
    """Evict every other sequence of the workload's batch to pinned host memory and bring it back
    (pa_bm_swap_out / pa_swap_blocks, then pa_bm_swap_in / pa_swap_blocks), timed with HIP events on
    the launch stream.  Bytes = pairs x layers x 2 pools x block bytes."""
    w = wl.WORKLOADS[args.workload]
    if args.block_size != w.block_size:
        w = w.replace(block_size=args.block_size, num_blocks=w.num_blocks * 16 // args.block_size)
    if args.num_blocks:
        w = w.replace(num_blocks=args.num_blocks)
    b = DecodeBatch(w, device="cuda", num_sets=1)
    torch.cuda.synchronize()
    caches = [b.caches[l] for l in b.layers]
    st = b.sets[0]
    victims = st.seqs[::2]
    need = sum(len(b.bm.table(s)) for s in victims)
    host = api.HostPools(caches, need)
    b.bm.set_host_blocks(need)
    out_pairs = np.concatenate([b.bm.swap_out(s) for s in victims]).astype(np.int32)
    in_pairs = np.concatenate([b.bm.swap_in(s) for s in victims]).astype(np.int32)
    d_out, d_in = torch.from_numpy(out_pairs).cuda(), torch.from_numpy(in_pairs).cuda()
    calls = {"out": api.SwapCall(caches, host, d_out, True),
             "in": api.SwapCall(caches, host, d_in, False)}
    stream = torch.cuda.current_stream()
    res = {}
    for name, call in calls.items():
        call()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        ev0.record(stream)
        for _ in range(reps):
            call()
        ev1.record(stream)
        torch.cuda.synchronize()
        sec = ev0.elapsed_time(ev1) / 1e3 / reps
        npairs = len(out_pairs) if name == "out" else len(in_pairs)
        nbytes = npairs * len(caches) * 2 * host.block_bytes
        res[name] = {"pairs": npairs, "bytes": nbytes, "us": round(sec * 1e6, 2),
                     "GB_per_s": round(nbytes / sec / 1e9, 2)}
    print(json.dumps({"metric": "swap to/from pinned host memory (pa_swap_blocks)",
                      "workload": f"{w.name}: every other sequence of the batch, unshared blocks",
                      "layers": len(caches), "block_bytes": host.block_bytes,
                      "swap_out": res["out"], "swap_in": res["in"]}), flush=True)
    return 0


def prefill_bench(args, torch, api, wl) -> int:
    """Prefill of S prompts of P tokens each: every token attends to the positions up to its own,
    through the block tables (pa_prefill_attention), timed with HIP events on the launch stream.
    Algorithmic flops = 4 * head_dim * num_q_heads * sum over tokens of the positions attended."""
    S, P = args.prefill
    Hq, H, D, B = 28, 4, 128, 16
    nb = S * (-(-P // B)) + 16
    w = wl.WORKLOADS["f16_batch32"].replace(num_seqs=S, num_blocks=nb)
    bm = api.BlockManager(nb, B, wl.free_order(w))
    seqs = [bm.add_seq() for _ in range(S)]
    slots = np.concatenate([bm.append_many(s, P) for s in seqs])
    tables, ctx = bm.export(seqs, -(-P // B), 0)
    g = wl.torch_generator(w.seed, "cuda")
    cache = api.KVCache.allocate(nb, H, D, "f16", "cuda")
    api.pa_reshape_and_cache(cache, wl.normal((S * P, H, D), "f16", g, "cuda"),
                             wl.normal((S * P, H, D), "f16", g, "cuda"),
                             torch.from_numpy(slots).cuda())
    q = wl.normal((S * P, Hq, D), "f16", g, "cuda")
    out = torch.empty_like(q)
    qs = torch.arange(0, S * P + 1, P, dtype=torch.int32, device="cuda")
    call = api.PrefillCall(out, q, cache, torch.from_numpy(tables).cuda(),
                           torch.from_numpy(ctx).cuda(), qs, P, P, 1.0 / math.sqrt(D))
    call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(1, args.steps)
    ev0.record(stream)
    for _ in range(reps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    sec = ev0.elapsed_time(ev1) / 1e3 / reps
    flops = 4.0 * D * Hq * S * (P * (P + 1) / 2)
    tflops = flops / sec / 1e12
    kv_bytes = S * P * 2 * H * D * 2
    print(json.dumps({
        "metric": "paged prefill attention (pa_prefill_attention)",
        "workload": f"{S} prompts x {P} tokens, 28 q / 4 KV heads, head_dim 128, f16, causal",
        "tokens_per_s": round(S * P / sec, 1), "us_per_call": round(sec * 1e6, 2),
        "calls_timed": reps,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(tflops / 2500.0, 4),
                     "flops_per_call": flops, "kv_bytes_written_before": kv_bytes}}), flush=True)
    return 0


def decode_call_mean(batch, torch, sets: int, n: int, flags: int = 0, fused: bool = False,
                     budget_s: float = 2e-3, first_reps: int = 3) -> float:
    """Mean duration of one decode call: n calls back to back (rotating over sets and layers), a
    few times over, between two HIP events on the stream they run on."""
    lay = list(batch.layers)

    def calls():
        for k in range(n):
            batch.decode(k % sets, lay[(k // sets) % len(lay)], flags=flags, append=fused)

    for _ in range(first_reps):
        calls()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    calls()
    torch.cuda.synchronize()
    est = (time.perf_counter() - t0) / n
    reps = max(1, min(20, int(budget_s / max(est, 1e-6))))
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(reps):
        calls()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / 1e3 / (reps * n)


def target_call(name: str, torch, api, wl, DecodeBatch) -> dict:
    """The decode call of another workload, measured in the same run: its roofline fraction."""
    w = wl.WORKLOADS[name]
    sets = DEFAULT_SETS[name]
    b = DecodeBatch(w, device="cuda", num_sets=sets)
    for r in range(sets):
        b.run_step(r)
    torch.cuda.synchronize()
    sec = decode_call_mean(b, torch, sets, max(8, min(64, sets * len(b.layers))))
    unique = w.prefix_len > 0
    alg = algorithmic_bytes(b, unique=unique)
    ach = alg / sec / 1e9
    out = {"workload": f"{w.name}: {w.description}", "decode_call_us": round(sec * 1e6, 3),
           "bytes_per_call": alg, "bytes_kind": "unique physical KV slots" if unique else
           "logical KV", "achieved": round(ach, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": round(ach / HBM_PEAK_GBPS, 4)}
    del b
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=list(DEFAULT_SETS))
    ap.add_argument("--passes", type=int, default=5,
                    help="passes of the timed loop (each times exactly --steps steps); value and "
                         "ms_per_step come from the median pass")
    ap.add_argument("--targets", default=None,
                    help="comma-separated workloads whose decode call is measured in the same run "
                         "(roofline only); default: the 32K-context batch beside the default "
                         "workload, none otherwise; '' for none")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--sets", type=int, default=0, help="independent batches rotated (0 = default)")
    ap.add_argument("--valu", action="store_true", help="force the vector-ALU decode kernel")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step as a captured HIP graph instead of launching every call "
                         "from Python")
    ap.add_argument("--partition", type=int, default=-1, help="partition size (-1 = workload's)")
    ap.add_argument("--num-blocks", type=int, default=0,
                    help="physical blocks per layer pool (0 = the workload's own)")
    ap.add_argument("--block-size", type=int, default=16, choices=(8, 16, 32),
                    help="token positions per block (pool of the same bytes: num_blocks scaled by "
                         "16 / block size)")
    ap.add_argument("--no-prefix", action="store_true",
                    help="shared-prefix workload: use the plain decode instead of the shared-prefix one")
    ap.add_argument("--contiguous", action="store_true",
                    help="control: physical blocks handed out in pool order, so that every "
                         "sequence's blocks are adjacent (the indirection-overhead baseline)")
    ap.add_argument("--fused", action="store_true",
                    help="step through pa_decode_attention_append (the cache write inside the "
                         "decode kernel) instead of reshape_and_cache + decode")
    ap.add_argument("--no-plan", action="store_true",
                    help="deal the decode's work in batch order instead of pa_decode_plan's order")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--swap", action="store_true",
                    help="measure swapping half of the workload's sequences to pinned host memory "
                         "and back (pa_swap_blocks), print that line and exit")
    ap.add_argument("--prefill", type=int, nargs=2, default=None, metavar=("SEQS", "PROMPT"),
                    help="measure paged prefill of SEQS prompts of PROMPT tokens each "
                         "(pa_prefill_attention, Qwen2.5-7B heads, f16), print that line and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB a few times (the "
                         "reference kernel for scaling HBM byte counters) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path here runs on a single MI355X and "
              "has no multi-GPU mode (sharding would split sequences, KV heads or context "
              "partitions across GPUs; it is not built).", file=sys.stderr)
        return 2

    import torch

    from paged_kv_cache_356_amd import api
    from paged_kv_cache_356_amd import workloads as wl
    from paged_kv_cache_356_amd.decode_batch import DecodeBatch

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        return 1
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n,
                          "copies": 3}), flush=True)
        return 0
    api.lib()
    if args.swap:
        return swap_bench(args, torch, api, wl, DecodeBatch)
    if args.prefill:
        return prefill_bench(args, torch, api, wl)
    w = wl.WORKLOADS[args.workload]
    if args.block_size != w.block_size:
        w = w.replace(block_size=args.block_size, num_blocks=w.num_blocks * 16 // args.block_size)
    if args.num_blocks:
        w = w.replace(num_blocks=args.num_blocks)
    sets = args.sets or DEFAULT_SETS[w.name]
    flags = api.PA_DECODE_FORCE_VALU if args.valu else api.PA_DECODE_DEFAULT
    t_build = time.perf_counter()
    batch = DecodeBatch(w, device="cuda", num_sets=sets,
                        keep_values=not args.no_cpu_baseline,
                        partition_size=None if args.partition < 0 else args.partition,
                        contiguous=args.contiguous,
                        keep_layers=[0], plan=not args.no_plan)
    batch.use_prefix = batch.use_prefix and not args.no_prefix
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: built {sets} set(s), {len(batch.layers)} layer(s) in "
        f"{time.perf_counter() - t_build:.1f} s; lengths {wl.lengths_summary(batch.lengths)}")

    layers = batch.layers
    # the planner's host time for one set (step metadata, computed beside the block tables)
    plan_us = None
    if not args.no_plan:
        st0 = batch.sets[0]

        def plan():
            api.pa_decode_plan(batch.caches[layers[0]], st0.q[layers[0]].dtype, st0.ctx,
                               w.num_q_heads, batch.max_blocks, batch.max_context_len,
                               batch.prefix_len if batch.use_prefix else 0, batch.partition_size,
                               (api.PA_DECODE_FORCE_VALU if args.valu else 0) |
                               (api.PA_DECODE_PLAN_APPEND if args.fused else 0))
        plan()  # the first call also queries the kernel's occupancy once per process
        t0 = time.perf_counter()
        for _ in range(20):
            plan()
        plan_us = round((time.perf_counter() - t0) / 20 * 1e6, 1)

    # Every library call enqueues on torch's current stream: the default stream when run eagerly,
    # the capture stream while a graph is being captured.
    fused = args.fused

    def step(r: int):
        """One step of set r: the copy-on-write clone, then per layer the new token's K/V write and
        the decode attention (one fused call with --fused, else reshape_and_cache + decode)."""
        batch.copy(r)
        for l in layers:
            if not fused:
                batch.reshape(r, l)
            batch.decode(r, l, flags=flags, append=fused)

    def decodes(n: int):
        """n decode calls back to back, rotating over sets and layers (fresh KV for each); the
        fused calls rewrite the step's token, the same bytes to the same slot each time."""
        for k in range(n):
            batch.decode(k % sets, layers[(k // sets) % len(layers)], flags=flags, append=fused)

    n_dec = max(8, min(64, sets * len(layers)))
    # Set-up: one pass over every set (the first write into a set's clone targets costs
    # milliseconds), then the W warm-up steps.
    for r in range(sets):
        step(r)
    torch.cuda.synchronize()
    for k in range(args.warmup):
        step(k % sets)
    decodes(n_dec)  # eager pass: first-call set-up happens outside any capture
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} step(s) done")
    if not args.graph:
        run_step = lambda k: step(k % sets)
        run_decodes = lambda: decodes(n_dec)
    else:
        # The step's launches replayed as one HIP graph per set.
        graphs = []
        for r in range(sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(r)
            graphs.append(g)
        g_dec = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_dec):
            decodes(n_dec)
        torch.cuda.synchronize()
        for r in range(sets):  # one untimed replay of each
            graphs[r].replay()
        g_dec.replay()
        torch.cuda.synchronize()
        run_step = lambda k: graphs[k % sets].replay()
        run_decodes = g_dec.replay
    # Python's cyclic garbage collector is run before the timed region and kept off during it (as
    # timeit does): a full collection takes tens of milliseconds, longer than many steps.
    gc.collect()
    gc.disable()
    pass_s = []
    for p in range(max(1, args.passes)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            run_step(k)
        torch.cuda.synchronize()
        pass_s.append(time.perf_counter() - t0)
        log(f"[bench] pass {p}: timed {args.steps} step(s) in {pass_s[-1] * 1e3:.2f} ms")
    elapsed = float(np.median(pass_s))

    # Decode-call duration for the roofline: n_dec calls back to back between two HIP events on the
    # stream they run on, a few times over.
    reps = max(1, min(20, int(2e-3 / max(elapsed / args.steps / len(layers), 1e-6))))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    ev0.record(stream)
    for _ in range(reps):
        run_decodes()
    ev1.record(stream)
    torch.cuda.synchronize()
    dec_mean_s = ev0.elapsed_time(ev1) / 1e3 / (reps * n_dec)

    # Per-call distributions: 20 repetitions of a batch of back-to-back eager calls, an event on
    # the launch stream around each batch (an event between single calls would add its own
    # ~2 us); p10 / p50 / p90 over the batches' per-call times.  The decode call, and the step's
    # other calls: reshape_and_cache (per layer) and copy_blocks (all layers at once, when the
    # step clones).
    lay = list(batch.layers)

    def per_call(fn, n: int, reps: int = 20):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        evs[0].record(stream)
        for r in range(reps):
            for k in range(n):
                fn(r * n + k)
            evs[r + 1].record(stream)
        torch.cuda.synchronize()
        us = np.array([evs[r].elapsed_time(evs[r + 1]) * 1e3 / n for r in range(reps)])
        return {"p10": round(float(np.percentile(us, 10)), 3), "p50": round(float(np.median(us)), 3),
                "p90": round(float(np.percentile(us, 90)), 3), "mean": round(float(us.mean()), 3),
                "calls": n * reps}

    n_pc = max(4, min(16, sets * len(lay)))
    dec_pc = per_call(lambda k: batch.decode(k % sets, lay[(k // sets) % len(lay)], flags=flags,
                                             append=fused), n_pc)
    resh_pc = None if fused else per_call(
        lambda k: batch.reshape(k % sets, lay[(k // sets) % len(lay)]), n_pc)
    copy_pc = per_call(lambda k: batch.copy(k % sets), max(4, sets)) \
        if batch.sets[0].pairs.shape[0] else None
    gc.enable()
    ms_per_step = elapsed * 1e3 / args.steps
    # the partition size the decode calls were made with (the planner's, where it picked one)
    call_partition = batch.call_partition(0, flags, fused) or batch.partition_size or \
        api.pa_decode_auto_partition(w.num_seqs, w.num_kv_heads, batch.max_context_len)
    layers = len(batch.layers)
    kv_logical = batch.kv_bytes_per_layer(unique=False)
    unique = w.prefix_len > 0
    alg = algorithmic_bytes(batch, unique=unique)
    if fused:  # the call also reads each new token's K/V row and writes it into the cache
        e_in = 4 if w.q_dtype == "f32" else 2
        e_c = 1 if w.cache_dtype == "fp8" else (4 if w.cache_dtype == "f32" else 2)
        alg += w.num_seqs * (2 * w.num_kv_heads * w.head_dim * (e_in + e_c) + 8)
    achieved = alg / dec_mean_s / 1e9
    kv_step = (batch.kv_bytes_per_layer(unique=True) if unique else kv_logical) * layers
    value = kv_step / (ms_per_step / 1e3) / 1e9
    seqs_per_s_layer = w.num_seqs / (ms_per_step / 1e3 / layers)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "passes_ms_per_step": [round(t * 1e3 / args.steps, 5) for t in pass_s],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.cache_dtype if w.cache_dtype != "fp8" else "fp8-e4m3 KV, f16 q",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": w.block_size, "layers": layers,
            "num_blocks_per_layer": w.num_blocks, "context_lens": wl.lengths_summary(batch.lengths),
            "partition_size": call_partition,
            "partition_planned": bool(not batch.partition_size and
                                      batch.call_partition(0, flags, fused)),
            "kernel": "valu" if args.valu else "default",
            "shared_prefix_decode": bool(batch.use_prefix),
            "dealing_order": "batch order" if args.no_plan else
                             "pa_decode_plan (host, from each set's context lengths)" if
                             batch.order(0, flags, fused) is not None else
                             "pa_decode_plan: the batch order itself for these lengths",
            "plan_host_us": plan_us,
            "block_placement": "contiguous (free list in pool order)" if args.contiguous else
                               "scattered (seeded permutation of the pool)",
            "step_calls": "copy_blocks (when the step clones) + per layer " +
                          ("pa_decode_attention_append (cache write fused into the decode kernel)"
                           if fused else "pa_reshape_and_cache + decode"),
            "sets_rotated": sets,
            "launch": "hip graph replay" if args.graph else "eager (GPU-bound)",
            "value_bytes": "unique physical KV slots per step (the shared prefix once)" if unique
                           else "logical KV bytes per step",
            "kv_bytes_per_step_logical": kv_logical * layers,
            "kv_bytes_per_layer_unique": batch.kv_bytes_per_layer(unique=True) if unique else
            kv_logical,
            "copy_pairs_per_step": int(batch.sets[0].pairs.shape[0]),
            # the block-size tradeoff: table entries the kernel reads, and positions allocated but
            # not (yet) used in each sequence's last block
            "table_entries_per_layer": int(sum(-(-int(L) // w.block_size) for L in batch.lengths)),
            "slots_allocated_unused": int(sum(-(-int(L) // w.block_size) * w.block_size - int(L)
                                              for L in batch.lengths)),
        },
        "hbm_fraction_of_step": round(value / HBM_PEAK_GBPS, 4),
        "seqs_per_s_per_layer": round(seqs_per_s_layer, 1),
        "decode_call_us_mean": round(dec_mean_s * 1e6, 3),
        "decode_call_us": dec_pc,
        "reshape_call_us": resh_pc,
        "copy_call_us": copy_pc,
        "seqs_per_s_per_layer_calls": round(w.num_seqs / (
            (dec_pc["p50"] + (resh_pc["p50"] if resh_pc else 0.0) +
             (copy_pc["p50"] / len(lay) if copy_pc else 0.0)) * 1e-6), 1),
        "decode_calls_timed": reps * n_dec,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(w, args.partition < 0 and not args.valu and not fused and
                                        not args.contiguous and not args.no_plan and
                                        not args.num_blocks and not args.no_prefix and
                                        args.block_size == 16, call_partition),
            "traffic_note": "HBM bytes per call from rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE "
                            "(decode + reduce kernels; profiles/traffic.json), null unless this run "
                            "is the measured configuration of unchanged kernels",
            "kernel": ("pa_decode_attention_append" + (" (shared prefix)" if batch.use_prefix else "")
                       if fused else "pa_decode_attention_shared_prefix" if batch.use_prefix else
                       "pa_decode_attention") + " (split-K decode + partition reduce)",
            "bytes_per_call": alg,
            "bytes_kind": "unique physical KV slots" if unique else "logical KV",
        },
    }
    if not args.no_calibration:
        res["calibration"] = calibration(batch, torch, api, sets)
        log(f"[bench] calibration {res['calibration']}")
    default_run = (args.workload == DEFAULT_WORKLOAD and not fused and not args.valu and
                   args.partition < 0 and args.block_size == 16 and not args.contiguous and
                   not args.no_prefix and not args.num_blocks and not args.no_plan)
    targets = args.targets if args.targets is not None else \
        ("bf16_32k_batch8" if default_run else "")
    if targets:
        res["targets"] = {}
        for name in [t for t in targets.split(",") if t]:
            res["targets"][name] = target_call(name, torch, api, wl, DecodeBatch)
            log(f"[bench] target {name}: {res['targets'][name]}")
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(batch, args.cpu_budget)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
