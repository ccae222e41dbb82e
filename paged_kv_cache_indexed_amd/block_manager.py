"""Host-side block manager: which physical blocks each sequence owns, and the device inputs
of one decode step.

It is "an address mapper, not an allocator" ([BlockManager essay] §2): it hands out ids
of a pool the caller preallocated, keeps one reference count per block, and turns the
state of a batch into the int32 arrays the library consumes:

  * ``block_table`` [batch][max_blocks_per_seq], -1 where unallocated ([BlockManager essay]
    §2, §5.1),
  * ``context_lens`` [batch] ([Valid-length essay] §4.1),
  * ``slot_mapping`` for appended tokens (slot = physical block * block_size + offset),
  * copy-on-write ``pairs`` (src, dst) for ``pa_copy_blocks``.

Rules from the pages:
  * allocate/free are O(1) on a free list ([KV Block course] §3.4); an empty pool raises
    ("Out of GPU blocks", [BlockManager essay] §5.1);
  * a request that would exceed max_blocks_per_seq is rejected, never written past the
    table ([BlockManager essay] §4.1);
  * blocks shared by several sequences (beam search) carry a reference count and return to
    the pool only at zero ([KV Block course] §3.4); every exit path releases them, including
    cancellation, through a context manager ([BlockManager essay] §4.2);
  * a sequence about to write into a block it shares gets a private copy first (copy-on-
    write); the sequence that forks keeps the original;
  * defragmentation moves the live blocks into one contiguous range of ids and rewrites the
    tables ([CANN paging article] §5.1); changing the block size needs a new layout and a
    migration of the contents ([CANN paging article] §4.1).
"""

from __future__ import annotations

import contextlib
from dataclasses import dataclass, field

import numpy as np


class OutOfBlocks(RuntimeError):
    """The pool has no free block."""


class BlockTableOverflow(ValueError):
    """A sequence would need more blocks than max_blocks_per_seq."""


@dataclass
class _Seq:
    blocks: list = field(default_factory=list)
    length: int = 0


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, max_blocks_per_seq: int,
                 shuffle_seed: int | None = None):
        if num_blocks <= 0 or block_size <= 0 or max_blocks_per_seq <= 0:
            raise ValueError("sizes must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.max_blocks_per_seq = int(max_blocks_per_seq)
        order = np.arange(self.num_blocks)
        if shuffle_seed is not None:
            order = np.random.default_rng(shuffle_seed).permutation(self.num_blocks)
        # pop() takes from the end: reverse so the first id handed out is order[0]
        self._free = [int(i) for i in order[::-1]]
        self.ref_count = np.zeros(self.num_blocks, np.int32)
        self._seqs: dict[int, _Seq] = {}

    # -------------------------------------------------------------- block level
    @property
    def num_free(self) -> int:
        return len(self._free)

    def allocate_block(self) -> int:
        if not self._free:
            raise OutOfBlocks("Out of GPU blocks")
        bid = self._free.pop()
        self.ref_count[bid] = 1
        return bid

    def release_block(self, bid: int) -> None:
        bid = int(bid)
        if not 0 <= bid < self.num_blocks or self.ref_count[bid] <= 0:
            raise ValueError(f"block {bid} is not allocated (double free?)")
        self.ref_count[bid] -= 1
        if self.ref_count[bid] == 0:
            self._free.append(bid)

    # -------------------------------------------------------------- sequences
    def add_sequence(self, seq_id: int) -> None:
        if seq_id in self._seqs:
            raise ValueError(f"sequence {seq_id} exists")
        self._seqs[seq_id] = _Seq()

    def fork(self, parent: int, child: int) -> None:
        """``child`` shares every block of ``parent`` (reference counts go up)."""
        if child in self._seqs:
            raise ValueError(f"sequence {child} exists")
        p = self._seqs[parent]
        for bid in p.blocks:
            self.ref_count[bid] += 1
        self._seqs[child] = _Seq(list(p.blocks), p.length)

    def free_sequence(self, seq_id: int) -> None:
        s = self._seqs.pop(seq_id)
        for bid in s.blocks:
            self.release_block(bid)

    @contextlib.contextmanager
    def sequence(self, seq_id: int):
        """Owns a sequence for the duration of a ``with`` block and frees it on every exit."""
        self.add_sequence(seq_id)
        try:
            yield seq_id
        finally:
            if seq_id in self._seqs:
                self.free_sequence(seq_id)

    def length(self, seq_id: int) -> int:
        return self._seqs[seq_id].length

    def blocks(self, seq_id: int) -> list:
        return list(self._seqs[seq_id].blocks)

    def copy_on_write(self, seq_id: int, logical_block: int) -> tuple[int, int] | None:
        """Give ``seq_id`` a private copy of its logical block if it is shared.

        Returns the (src, dst) pair to pass to pa_copy_blocks, or None if the block was
        already private. The other sharers keep the original block.
        """
        s = self._seqs[seq_id]
        src = s.blocks[logical_block]
        if self.ref_count[src] <= 1:
            return None
        dst = self.allocate_block()
        self.ref_count[src] -= 1
        s.blocks[logical_block] = dst
        return (src, dst)

    def append_slots(self, seq_id: int, n: int = 1):
        """Reserve slots for ``n`` new tokens at the end of ``seq_id``.

        Returns (slots, cow_pairs). A new block is allocated when the last one is full; a
        shared, partly filled last block is copied first. Rejects the request, changing
        nothing, if the sequence would exceed max_blocks_per_seq.
        """
        s = self._seqs[seq_id]
        bs = self.block_size
        need = -(-(s.length + n) // bs)
        if need > self.max_blocks_per_seq:
            raise BlockTableOverflow(
                f"sequence {seq_id} needs {need} blocks > max_blocks_per_seq {self.max_blocks_per_seq}")
        new_blocks = need - len(s.blocks)
        cow_needed = s.length % bs != 0 and self.ref_count[s.blocks[-1]] > 1
        if new_blocks + int(cow_needed) > self.num_free:
            raise OutOfBlocks("Out of GPU blocks")
        pairs = []
        if cow_needed:
            pairs.append(self.copy_on_write(seq_id, len(s.blocks) - 1))
        slots = []
        for t in range(s.length, s.length + n):
            j, off = divmod(t, bs)
            if j == len(s.blocks):
                s.blocks.append(self.allocate_block())
            slots.append(s.blocks[j] * bs + off)
        s.length += n
        return np.array(slots, np.int32), pairs

    # -------------------------------------------------------------- maintenance
    def num_live(self) -> int:
        return int(np.count_nonzero(self.ref_count))

    def is_compact(self) -> bool:
        """Every live block has an id below the number of live blocks."""
        return bool(np.all(self.ref_count[self.num_live():] == 0))

    def compact(self) -> np.ndarray:
        """Defragment: move every live block with an id >= the number of live blocks into a
        free id below it ([CANN paging article] §5.1: compact the active blocks into one
        region, then update the mapping), and rewrite the tables and reference counts.

        Returns int32 pairs (src, dst) for pa_copy_blocks. Every dst is free and every src is
        live, so the pairs may run in parallel; the device copy must complete before the new
        tables (block_table) are used, and the moved sources are free afterwards. Afterwards
        the free list hands out the lowest ids first.
        """
        n_live = self.num_live()
        movers = [int(i) for i in np.nonzero(self.ref_count[n_live:])[0] + n_live]
        holes = [int(i) for i in np.nonzero(self.ref_count[:n_live] == 0)[0]]
        assert len(movers) == len(holes)
        mapping = dict(zip(movers, holes))
        for s in self._seqs.values():
            s.blocks = [mapping.get(b, b) for b in s.blocks]
        for src, dst in mapping.items():
            self.ref_count[dst] = self.ref_count[src]
            self.ref_count[src] = 0
        self._free = list(range(self.num_blocks - 1, n_live - 1, -1))
        return np.array(list(mapping.items()), np.int32).reshape(-1, 2)

    def reblocked(self, block_size: int, num_blocks: int | None = None,
                  max_blocks_per_seq: int | None = None) -> "BlockManager":
        """A manager for a new pool of another block size that holds the same sequences with
        the same lengths ([CANN paging article] §4.1). Each sequence gets private blocks in
        the new pool (blocks of two sizes do not line up, so sharing is not carried over).
        Pass both managers' block_table() for the same sequence order to pa_reblock.
        """
        bs = int(block_size)
        need = {sid: -(-s.length // bs) for sid, s in self._seqs.items()}
        nb = int(num_blocks) if num_blocks is not None else max(1, sum(need.values()))
        mbs = int(max_blocks_per_seq) if max_blocks_per_seq is not None else max([1, *need.values()])
        new = BlockManager(nb, bs, mbs)
        for sid, s in self._seqs.items():
            new.add_sequence(sid)
            if s.length:
                new.append_slots(sid, s.length)
        return new

    # -------------------------------------------------------------- device inputs
    def block_table(self, seq_ids) -> np.ndarray:
        t = np.full((len(seq_ids), self.max_blocks_per_seq), -1, np.int32)
        for r, sid in enumerate(seq_ids):
            b = self._seqs[sid].blocks
            t[r, :len(b)] = b
        return t

    def context_lens(self, seq_ids) -> np.ndarray:
        return np.array([self._seqs[s].length for s in seq_ids], np.int32)

    def check_invariants(self) -> None:
        """free + used == total, and every reference is held by some table entry."""
        held = np.zeros(self.num_blocks, np.int64)
        for s in self._seqs.values():
            for bid in s.blocks:
                held[bid] += 1
        assert np.array_equal(held, self.ref_count), "reference counts != table entries"
        used = int(np.count_nonzero(self.ref_count))
        assert used + len(self._free) == self.num_blocks, "free + used != total"
        assert len(set(self._free)) == len(self._free), "duplicate free id"
        assert all(self.ref_count[i] == 0 for i in self._free), "free block still referenced"
