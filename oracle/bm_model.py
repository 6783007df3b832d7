"""TEST INFRASTRUCTURE ONLY — a plain model of the paged KV block manager.

It follows the pages step by step:
  * a shared pool of fixed-size physical blocks; blocks are handed out as sequences grow and go back
    to the pool when a sequence finishes ("PagedAttention" (devoured.fyi), "PagedAttention in one
    picture");
  * a per-sequence block table mapping logical block index to physical block id (same section);
  * a new block is mapped only when the previous one is full; each token takes the next slot of
    the sequence's last block ("LLM Inference Visualizer, Lesson 06", "How paging grows");
  * shared blocks carry a reference count; fork shares every block ("PagedAttention, Visualized",
    Part 3, copy-on-write after fork / shared prefix blocks);
  * a write into a block whose count is above 1 clones it, decrements the original and retargets the
    writer's table ("PagedAttention" (devoured.fyi), "Copy-on-write: when two requests share a
    prefix");
  * swapping to disk is, for the KV cache, evicting blocks to CPU memory; when a sequence is
    evicted, its shared blocks do not move, because another sequence still needs them ("PagedAttention,
    Visualized", Part 3, the OS-to-PagedAttention table and the paragraph after it).

Readings where the pages are silent (also listed with the other readings of the build):
  * the free list is a stack: the caller gives the initial order (its first entry is handed out
    first) and a freed block is pushed on top, to be handed out next;
  * sequence ids count up from 0 and are never reused;
  * on an empty free list an append changes nothing and reports exhaustion;
  * CPU memory is a pool of host slots with a stack of its own, handed out 0, 1, 2, ... at first;
  * swapping a sequence out moves exactly its blocks whose count is 1, in table order, each to a
    fresh host slot, and frees those device blocks; a shared block stays on the device and the
    evicted sequence keeps its reference to it, so it cannot be freed meanwhile;
  * swapping it in takes one device block per host slot, in table order, and frees the slots;
  * both report the moves as (device block, host slot) pairs, and change nothing (and report
    exhaustion) when there are too few free host slots or device blocks for the whole sequence;
  * a swapped-out sequence cannot append, fork or be exported until it is swapped in; it can be
    freed, which returns its host slots.
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
        self.host_free: list[int] = []        # top of the stack is the end of the list
        self.num_host = 0
        self.on_host: dict[int, list[bool]] = {}  # per swapped-out sequence: entry is a host slot

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
        assert parent not in self.on_host, "a swapped-out sequence cannot fork"
        child = self.add_seq()
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1
        return child

    def append(self, seq: int):
        """Returns (slot, cow) where cow is (src, dst) or None."""
        assert seq not in self.on_host, "a swapped-out sequence cannot append"
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
        where = self.on_host.pop(seq, None)
        for j, b in enumerate(self.tables.pop(seq)):
            if where is not None and where[j]:
                self.host_free.append(b)
            else:
                self._release(b)
        del self.lens[seq]

    # -- swapping to CPU memory
    def set_host_blocks(self, n: int) -> None:
        assert not self.on_host, "host slots are in use"
        self.num_host = n
        self.host_free = list(reversed(range(n)))

    def swap_out(self, seq: int):
        """Evict seq: its unshared blocks go to host slots.  Returns [(device block, host slot)]."""
        assert seq not in self.on_host
        table = self.tables[seq]
        move = [j for j, b in enumerate(table) if self.ref[b] == 1]
        if len(move) > len(self.host_free):
            raise NoBlocks()
        where = [False] * len(table)
        pairs = []
        for j in move:
            b = table[j]
            h = self.host_free.pop()
            pairs.append((b, h))
            self._release(b)
            table[j] = h
            where[j] = True
        self.on_host[seq] = where
        return pairs

    def swap_in(self, seq: int):
        """Bring seq back: one device block per host slot.  Returns [(device block, host slot)]."""
        where = self.on_host[seq]
        table = self.tables[seq]
        move = [j for j in range(len(table)) if where[j]]
        if len(move) > len(self.free):
            raise NoBlocks()
        pairs = []
        for j in move:
            h = table[j]
            b = self._take()
            pairs.append((b, h))
            self.host_free.append(h)
            table[j] = b
        del self.on_host[seq]
        return pairs

    # -- views
    def table(self, seq: int) -> list[int]:
        return list(self.tables[seq])

    def export(self, seqs, max_blocks: int, pad: int):
        rows, lens = [], []
        for s in seqs:
            assert s not in self.on_host, "a swapped-out sequence has no device table"
            t = self.tables[s]
            assert len(t) <= max_blocks
            rows.append(t + [pad] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return rows, lens

    def check_invariants(self) -> None:
        """Counts equal the number of table entries naming each block; every block is either free
        or referenced, never both; each table holds exactly ceil(L / B) blocks."""
        count = [0] * self.num_blocks
        host_used = []
        for s, t in self.tables.items():
            assert len(t) == -(-self.lens[s] // self.block_size)
            where = self.on_host.get(s, [False] * len(t))
            for b, h in zip(t, where):
                if h:
                    host_used.append(b)
                else:
                    count[b] += 1
        assert count == self.ref
        free = set(self.free)
        assert len(free) == len(self.free)
        for b in range(self.num_blocks):
            assert (b in free) == (self.ref[b] == 0)
        # every host slot is used by exactly one swapped-out entry or free, never both
        assert sorted(host_used + self.host_free) == list(range(self.num_host))
