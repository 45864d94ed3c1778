"""Plain-Python model of the host block allocator (reference for its tests).

TEST INFRASTRUCTURE ONLY: nothing on the product path imports it; it shares
no code with the C++ allocator in the library.

What it models, and where that comes from
-----------------------------------------
* The paged cache's blocks are handed out on demand from a queue of free
  block ids kept on the host; a request that needs more room takes the next
  free block from the queue (Inference Engineering, Day 11 post on vLLM's KV
  cache manager and its free-block queue).
* Each sequence owns a block table and holds just enough blocks for its
  tokens, so the memory it wastes is less than one block (nanoserve
  write-up, "What I built", paged KV cache item).
* A chunk of a prompt fills the sequence's blocks in order (Inference
  Engineering, Day 12 post: 8-token chunks into 4-token blocks occupy 2
  blocks after one pass, 4 after two).

Readings where the pages are silent: the queue starts as 0..num_blocks-1; a
freed sequence's blocks go to the back of the queue in table order; a request
that does not fit changes nothing.
"""
from __future__ import annotations

from collections import deque


class NoSpace(Exception):
    """Not enough free blocks, or a table would pass its capacity."""


class BlockAllocatorRef:
    def __init__(self, num_blocks: int, block_size: int, max_seqs: int,
                 max_blocks_per_seq: int):
        self.block_size = block_size
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free = deque(range(num_blocks))
        self.tables = [[] for _ in range(max_seqs)]
        self.lens = [0] * max_seqs

    def _blocks_for(self, n_tokens: int) -> int:
        return -(-n_tokens // self.block_size)

    def _extra_blocks(self, seq: int, n: int) -> int:
        want = self._blocks_for(self.lens[seq] + n)
        if want > self.max_blocks_per_seq:
            raise NoSpace(f"sequence {seq} would need {want} blocks")
        return want - len(self.tables[seq])

    def slot_of(self, seq: int, pos: int) -> int:
        bs = self.block_size
        return self.tables[seq][pos // bs] * bs + pos % bs

    def append_slots(self, seq: int, n: int):
        if self._extra_blocks(seq, n) > len(self.free):
            raise NoSpace("free queue too short")
        want = self._blocks_for(self.lens[seq] + n)
        while len(self.tables[seq]) < want:
            self.tables[seq].append(self.free.popleft())
        first = self.lens[seq]
        self.lens[seq] += n
        return [self.slot_of(seq, p) for p in range(first, first + n)]

    def free_seq(self, seq: int):
        self.free.extend(self.tables[seq])
        self.tables[seq] = []
        self.lens[seq] = 0

    def block_table(self, seq: int, width: int):
        t = self.tables[seq]
        if width < len(t):
            raise ValueError("width below the table's blocks")
        return t + [-1] * (width - len(t))

    def _check_batch(self, seqs, counts, width):
        """Validates sequence by sequence, in batch order: a repeated id or a
        negative count, then the table's capacity, then the output width; the
        free queue is checked for the whole batch last."""
        seen = set()
        total = 0
        for s, n in zip(seqs, counts):
            if s in seen or n < 0:
                raise ValueError("repeated sequence id or negative count")
            seen.add(s)
            total += self._extra_blocks(s, n)
            if self._blocks_for(self.lens[s] + n) > width:
                raise ValueError("width below a table's blocks")
        if total > len(self.free):
            raise NoSpace("free queue too short for the batch")

    def decode_batch(self, seqs, width):
        """One new token per sequence: (slots, tables, context lengths)."""
        self._check_batch(seqs, [1] * len(seqs), width)
        slots = [self.append_slots(s, 1)[0] for s in seqs]
        return slots, [self.block_table(s, width) for s in seqs], [self.lens[s] for s in seqs]

    def prefill_batch(self, seqs, chunk_lens, width):
        """One chunk per sequence: (query_start, slots, tables, lengths)."""
        self._check_batch(seqs, chunk_lens, width)
        qs = [0]
        slots = []
        for s, n in zip(seqs, chunk_lens):
            slots += self.append_slots(s, n)
            qs.append(qs[-1] + n)
        return qs, slots, [self.block_table(s, width) for s in seqs], [self.lens[s] for s in seqs]
