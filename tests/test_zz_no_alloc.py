"""pa_decode_attention_noalloc (the decode with its partials in the library's fixed device scratch,
for callers that cannot allocate) against pa_decode_attention with a workspace: the same kernels on
the same partition sizes, so the outputs must be bitwise equal.  Two calls in a row, the second with
a smaller batch (the scratch keeps the first call's partials, which the second must never read)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from paged_kv_cache_356_amd import api
from paged_kv_cache_356_amd import workloads as wl
from paged_kv_cache_356_amd.decode_batch import DecodeBatch


def test_no_alloc_oversized_call_is_refused_before_any_device_work():
    """A call whose partials exceed the fixed scratch returns PA_ERR_WORKSPACE from host arithmetic
    alone (runs on the CPU too: no device is touched)."""
    c = api.pa_cache(16, 32, None, None, 8, 16, 4, 128, api.PA_F16)
    # 4,000 sequences x 28 heads x 32,768 positions in partitions of 16: far past 64 MiB
    st = api.lib().pa_decode_attention_noalloc(64, 128, api.PA_F16, 0, ctypes.byref(c), 256, 2048,
                                               512, 4000, 28, 32768, 0.1, 16, 0, None)
    assert st == -4
    assert "scratch" in api.lib().pa_last_error().decode()


@pytest.mark.gpu
def test_no_alloc_matches_the_workspace_decode_on_two_calls():
    torch.cuda.set_device(0)
    paired = [2600, 1, 257, 512, 513, 2599] + [100 + 83 * i for i in range(24)]
    cases = [
        # a batch whose items the kernel pairs (30 x 4 rows of up to 11 partitions: between one
        # and two items per SIMD on 256 compute units), then smaller ones
        ("f16_batch32", dict(num_seqs=30, num_blocks=8192), paired, 256),
        # several partitions per row (the partials live in the scratch), then a smaller batch
        ("f16_batch32", dict(num_seqs=12, num_blocks=2048), [2048, 1500, 700, 1, 17, 129, 256,
                                                            257, 1999, 64, 640, 1024], 128),
        ("f16_batch32", dict(num_seqs=3, num_blocks=2048), [900, 33, 512], 128),
    ]
    for name, kw, lengths, ps in cases:
        w = wl.WORKLOADS[name].replace(**kw)
        print(f"no-alloc decode: {w.num_seqs} sequences, lengths {lengths}", flush=True)
        b = DecodeBatch(w, pad_block=0, lengths=lengths, partition_size=ps)
        b.run_step(0)
        torch.cuda.synchronize()
        st = b.sets[0]
        ref = st.out[0].clone()
        got = torch.full_like(ref, float("nan"))
        api.pa_decode_attention_noalloc(got, st.q[0], b.caches[0], st.d_tables, st.d_ctx,
                                        b.max_context_len, w.scale, ps)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, ref), float((got.float() - ref.float()).abs().max())
