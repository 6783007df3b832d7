"""TEST INFRASTRUCTURE ONLY — a plain model of the paged KV block manager.

It follows the pages step by step:
  * a shared pool of fixed-size physical blocks; blocks are handed out as sequences grow and go back
    to the pool when a sequence finishes ("PagedAttention" (devoured.fyi), "PagedAttention in one
    picture");
  * a per-sequence block table mapping logical block index to physical block id (same section);
  * a new block is mapped only when the previous one is full; every token appends one entry in the
    current block ("LLM Inference Visualizer, Lesson 06", "How paging grows");
  * shared blocks carry a reference count; fork shares every block ("PagedAttention, Visualized",
    Part 3, copy-on-write after fork / shared prefix blocks);
  * a write into a block whose count is above 1 clones it, decrements the original and retargets the
    writer's table ("PagedAttention" (devoured.fyi), "Copy-on-write: when two requests share a
    prefix").

Readings where the pages are silent (also listed with the other readings of the build):
  * the free list is a stack: the caller gives the initial order (its first entry is handed out
    first) and a freed block is pushed on top, to be handed out next;
  * sequence ids count up from 0 and are never reused;
  * on an empty free list an append changes nothing and reports exhaustion.
"""
from __future__ import annotations


class NoBlocks(Exception):
    pass


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        assert sorted(order) == list(range(num_blocks)), "free_order must be a permutation"
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(reversed(order))  # top of the stack is the end of the list
        self.ref = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.next_id = 0

    # -- pool
    def _take(self) -> int:
        if not self.free:
            raise NoBlocks()
        b = self.free.pop()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        assert self.ref[b] >= 0
        if self.ref[b] == 0:
            self.free.append(b)

    # -- sequences
    def add_seq(self) -> int:
        s = self.next_id
        self.next_id += 1
        self.tables[s] = []
        self.lens[s] = 0
        return s

    def fork(self, parent: int) -> int:
        child = self.add_seq()
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1
        return child

    def append(self, seq: int):
        """Returns (slot, cow) where cow is (src, dst) or None."""
        B = self.block_size
        table = self.tables[seq]
        L = self.lens[seq]
        j, off = divmod(L, B)
        cow = None
        if off == 0:
            table.append(self._take())
        else:
            last = table[j]
            if self.ref[last] > 1:
                dst = self._take()           # clone target
                self.ref[last] -= 1          # the original loses this writer
                table[j] = dst               # the writer now points at the clone
                cow = (last, dst)
        self.lens[seq] = L + 1
        return table[j] * B + off, cow

    def append_batch(self, seqs):
        slots, pairs = [], []
        for s in seqs:
            slot, cow = self.append(s)
            slots.append(slot)
            if cow is not None:
                pairs.append(cow)
        return slots, pairs

    def free_seq(self, seq: int) -> None:
        for b in self.tables.pop(seq):
            self._release(b)
        del self.lens[seq]

    # -- views
    def table(self, seq: int) -> list[int]:
        return list(self.tables[seq])

    def export(self, seqs, max_blocks: int, pad: int):
        rows, lens = [], []
        for s in seqs:
            t = self.tables[s]
            assert len(t) <= max_blocks
            rows.append(t + [pad] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return rows, lens

    def check_invariants(self) -> None:
        """Counts equal the number of table entries naming each block; every block is either free
        or referenced, never both; each table holds exactly ceil(L / B) blocks."""
        count = [0] * self.num_blocks
        for s, t in self.tables.items():
            assert len(t) == -(-self.lens[s] // self.block_size)
            for b in t:
                count[b] += 1
        assert count == self.ref
        free = set(self.free)
        assert len(free) == len(self.free)
        for b in range(self.num_blocks):
            assert (b in free) == (self.ref[b] == 0)
