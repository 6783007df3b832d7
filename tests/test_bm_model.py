"""Pins for the oracle's block-manager model against what the pages state: blocks only when the
previous one is full, waste below one block, the external-fragmentation case, the copy-on-write
procedure, and the reference-count invariants under random operation sequences.  CPU only."""
from __future__ import annotations

import numpy as np
import pytest

from oracle.bm_model import BlockManagerModel, NoBlocks


def test_47_tokens_take_three_blocks():
    # "PagedAttention" (devoured.fyi), "PagedAttention in one picture": 47 tokens -> 3 blocks (48 slots)
    bm = BlockManagerModel(8, 16)
    s = bm.add_seq()
    for _ in range(47):
        bm.append(s)
    assert len(bm.table(s)) == 3 and 3 * 16 - 47 == 1


def test_waste_is_below_one_block_for_any_length():
    g = np.random.default_rng(0)
    bm = BlockManagerModel(4096, 16)
    for L in g.integers(1, 1000, 40):
        s = bm.add_seq()
        for _ in range(int(L)):
            bm.append(s)
        assert 0 <= 16 * len(bm.table(s)) - L <= 15


def test_blocks_are_mapped_only_when_the_previous_one_is_full():
    bm = BlockManagerModel(4, 4, free_order=[2, 0, 3, 1])
    s = bm.add_seq()
    grown = []
    for _ in range(9):
        before = len(bm.table(s))
        bm.append(s)
        grown.append(len(bm.table(s)) - before)
    assert grown == [1, 0, 0, 0, 1, 0, 0, 0, 1]
    assert bm.table(s) == [2, 0, 3]  # handed out in the caller's free-list order


def test_external_fragmentation_case_is_served_by_paging():
    # Lesson 06 "Why reservation fails": 3 free slots, no 3 adjacent; a paged manager (one slot per
    # page here) still serves a request needing 3 slots.
    bm = BlockManagerModel(6, 1)
    a, b, c = bm.add_seq(), bm.add_seq(), bm.add_seq()
    fill = [a, None, b, None, c, None]
    holders = {}
    for page, who in enumerate(fill):
        s = who if who is not None else bm.add_seq()
        bm.append(s)
        holders[page] = s
    for page in (1, 3, 5):
        bm.free_seq(holders[page])
    d = bm.add_seq()
    slots = [bm.append(d)[0] for _ in range(3)]
    assert sorted(slots) == [1, 3, 5]


def test_copy_on_write_procedure():
    # "PagedAttention" (devoured.fyi), copy-on-write: clone the shared block, decrement the
    # original's count, retarget the writer's table; everyone else keeps the original.
    bm = BlockManagerModel(8, 4)
    p = bm.add_seq()
    for _ in range(6):
        bm.append(p)
    c = bm.fork(p)
    assert bm.table(c) == bm.table(p) and all(bm.ref[b] == 2 for b in bm.table(p))
    shared_last = bm.table(p)[1]
    slot, cow = bm.append(c)
    assert cow is not None and cow[0] == shared_last
    assert bm.table(c)[1] == cow[1] != shared_last and bm.table(p)[1] == shared_last
    assert bm.ref[shared_last] == 1 and bm.ref[cow[1]] == 1 and bm.ref[bm.table(p)[0]] == 2
    assert slot == cow[1] * 4 + 2
    # the parent now owns its block alone and writes in place
    slot, cow = bm.append(p)
    assert cow is None and slot == shared_last * 4 + 2
    bm.check_invariants()


def test_fresh_block_needs_no_clone_even_when_shared():
    bm = BlockManagerModel(8, 4)
    p = bm.add_seq()
    for _ in range(4):
        bm.append(p)
    c = bm.fork(p)
    slot, cow = bm.append(c)  # position 4 opens a new block: nothing shared is written
    assert cow is None and bm.table(c)[0] == bm.table(p)[0] and bm.ref[bm.table(p)[0]] == 2


def test_exhaustion_changes_nothing():
    bm = BlockManagerModel(2, 2)
    s = bm.add_seq()
    for _ in range(4):
        bm.append(s)
    t = bm.fork(s)
    before = (bm.table(s), bm.table(t), list(bm.ref), list(bm.free), dict(bm.lens))
    with pytest.raises(NoBlocks):
        bm.append(s)   # needs a fresh block
    after = (bm.table(s), bm.table(t), list(bm.ref), list(bm.free), dict(bm.lens))
    assert before == after


def test_freed_blocks_are_reused_first():
    bm = BlockManagerModel(6, 2)
    a = bm.add_seq()
    for _ in range(4):
        bm.append(a)
    assert bm.table(a) == [0, 1]
    bm.free_seq(a)
    b = bm.add_seq()
    bm.append(b)
    assert bm.table(b) == [1]  # the last block released is on top of the stack


@pytest.mark.parametrize("seed", range(6))
def test_random_operation_sequences_keep_the_invariants(seed):
    g = np.random.default_rng(seed)
    bm = BlockManagerModel(64, 4, free_order=g.permutation(64))
    live = []
    for _ in range(600):
        op = g.integers(0, 10)
        try:
            if op == 0 or not live:
                live.append(bm.add_seq())
            elif op == 1:
                live.append(bm.fork(live[g.integers(len(live))]))
            elif op == 2 and len(live) > 1:
                bm.free_seq(live.pop(g.integers(len(live))))
            else:
                s = live[g.integers(len(live))]
                slot, cow = bm.append(s)
                t = bm.table(s)
                L = bm.lens[s]
                assert slot == t[(L - 1) // 4] * 4 + (L - 1) % 4
                assert bm.ref[t[(L - 1) // 4]] == 1  # the block written is never shared
                if cow is not None:
                    assert bm.ref[cow[0]] >= 1
        except NoBlocks:
            pass
        bm.check_invariants()


# --------------------------------------------------------------------------- swapping to CPU memory
# "PagedAttention, Visualized", Part 3: swapping to disk is evicting blocks to CPU memory, and an
# evicted sequence's shared blocks do not move, because another sequence still needs them.

def _shared_prompt_batch():
    """Two users share a 2-block prompt (block size 2, 4 tokens); each then adds 3 tokens of its
    own.  Free order 0..9: prompt blocks 0, 1; user a's own blocks 2, 3; user b's 4, 5."""
    bm = BlockManagerModel(10, 2)
    bm.set_host_blocks(3)
    p = bm.add_seq()
    for _ in range(4):
        bm.append(p)
    a, b = bm.fork(p), bm.fork(p)
    bm.free_seq(p)
    for s in (a, b):
        for _ in range(3):
            bm.append(s)
    return bm, a, b


def test_swap_out_moves_only_the_unshared_blocks():
    bm, a, b = _shared_prompt_batch()
    assert bm.table(a) == [0, 1, 2, 3] and bm.table(b) == [0, 1, 4, 5]
    pairs = bm.swap_out(a)
    # the prompt blocks 0, 1 stay (b still needs them); a's own blocks go to host slots 0, 1
    assert pairs == [(2, 0), (3, 1)]
    assert bm.ref[0] == bm.ref[1] == 2 and bm.ref[2] == bm.ref[3] == 0
    assert bm.free[-2:] == [2, 3]  # freed device blocks are next to be handed out (3 first)
    assert bm.host_free == [2]
    bm.check_invariants()
    # b runs on: its 8th token fills its block 5, its 9th opens a new block, the one a freed last
    assert bm.append(b) == (5 * 2 + 1, None)
    assert bm.append(b) == (3 * 2 + 0, None)
    assert bm.table(b) == [0, 1, 4, 5, 3]
    bm.check_invariants()


def test_swap_in_takes_fresh_device_blocks_in_table_order():
    bm, a, b = _shared_prompt_batch()
    bm.swap_out(a)
    pairs = bm.swap_in(a)
    # device blocks come off the free stack (3 on top, then 2); host slots 0, 1 are freed
    assert pairs == [(3, 0), (2, 1)]
    assert bm.table(a) == [0, 1, 3, 2]
    assert sorted(bm.host_free) == [0, 1, 2]
    bm.check_invariants()
    # a runs on from where it was: its 7th token continues its last block
    slot, cow = bm.append(a)
    assert slot == 2 * 2 + 1 and cow is None


def test_evicting_a_fully_shared_sequence_moves_nothing():
    bm = BlockManagerModel(8, 4)
    bm.set_host_blocks(2)
    p = bm.add_seq()
    for _ in range(8):
        bm.append(p)
    users = [bm.fork(p) for _ in range(3)]
    assert bm.swap_out(users[0]) == []
    assert bm.ref[bm.table(p)[0]] == 4
    assert bm.swap_in(users[0]) == []
    bm.check_invariants()


def test_swap_exhaustion_changes_nothing():
    bm, a, b = _shared_prompt_batch()
    bm.set_host_blocks(1)  # one slot, a needs two
    before = (bm.table(a), list(bm.ref), list(bm.free), list(bm.host_free))
    with pytest.raises(NoBlocks):
        bm.swap_out(a)
    assert before == (bm.table(a), list(bm.ref), list(bm.free), list(bm.host_free))
    bm.set_host_blocks(2)
    bm.swap_out(a)
    while bm.free:  # fill the device pool
        bm.append(bm.add_seq())
    before = (bm.tables[a][:], list(bm.ref), list(bm.host_free))
    with pytest.raises(NoBlocks):
        bm.swap_in(a)
    assert before == (bm.tables[a], list(bm.ref), list(bm.host_free))
    bm.check_invariants()


def test_freeing_a_swapped_out_sequence_returns_its_host_slots():
    bm, a, b = _shared_prompt_batch()
    bm.swap_out(a)
    bm.free_seq(a)
    assert sorted(bm.host_free) == [0, 1, 2]
    assert bm.ref[0] == bm.ref[1] == 1  # b alone holds the prompt now
    bm.check_invariants()


def test_a_swapped_out_sequence_cannot_run():
    bm, a, b = _shared_prompt_batch()
    bm.swap_out(a)
    for op in (lambda: bm.append(a), lambda: bm.fork(a), lambda: bm.export([a], 8, -1)):
        with pytest.raises(AssertionError):
            op()


@pytest.mark.parametrize("seed", range(6))
def test_random_sequences_with_swapping_keep_the_invariants(seed):
    g = np.random.default_rng(50 + seed)
    bm = BlockManagerModel(48, 4, free_order=g.permutation(48))
    bm.set_host_blocks(24)
    live, out = [], set()
    for _ in range(800):
        op = g.integers(0, 12)
        try:
            if op == 0 or not live:
                live.append(bm.add_seq())
            elif op == 1 and live:
                s = live[g.integers(len(live))]
                if s not in out:
                    live.append(bm.fork(s))
            elif op == 2 and len(live) > 1:
                s = live.pop(g.integers(len(live)))
                bm.free_seq(s)
                out.discard(s)
            elif op == 3:
                s = live[g.integers(len(live))]
                if s not in out:
                    moved = bm.swap_out(s)
                    out.add(s)
                    assert all(bm.ref[d] == 0 for d, _ in moved)
            elif op == 4 and out:
                s = sorted(out)[g.integers(len(out))]
                bm.swap_in(s)
                out.discard(s)
            else:
                s = live[g.integers(len(live))]
                if s not in out:
                    bm.append(s)
        except NoBlocks:
            pass
        bm.check_invariants()
