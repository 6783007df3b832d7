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
