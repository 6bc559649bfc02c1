"""Host-side block manager: the free pool, refcounted sharing and slot assignment.

This is the host step in front of the kernels: it decides which physical
16-token block each logical block of a sequence lives in, and which slot
each new token is written to.  It follows

* Habr KV-Cache article (habr.com/ru/articles/1021832), §4 "Recalling
  PagedAttention": fixed blocks of 16 tokens; a block table maps logical
  blocks to physical ones; the worked example (a 1024-token prompt plus 10
  generated tokens) opens a fresh block when the last one is full, so a
  sequence wastes at most one partial block; blocks shared by several
  sequences are reference counted, and a sequence that must modify a shared
  block copies it first (copy-on-write).
* Same article, §7 ("Cache Read"): full blocks are immutable and new decode
  tokens always go to fresh blocks; blocks whose count drops to zero return
  to the free pool.
* "Why one character breaks the cache", section on PagedAttention as
  virtual memory: each block carries a ref_cnt of the requests holding it.

Slots are flat, 0-based: ``slot = physical_block * block_size + offset``.  The
manager is single-threaded by design (the same article, §8, explains why a
single-threaded scheduler needs no locks around the table).
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Iterable, List, Optional, Tuple

import numpy as np

BLOCK_SIZE = 16


class OutOfBlocks(RuntimeError):
    """The free pool is empty."""


class SharedBlockWrite(RuntimeError):
    """A write would land in a block other sequences still reference."""


@dataclass
class _Sequence:
    blocks: List[int] = field(default_factory=list)
    num_tokens: int = 0


class BlockManager:
    """Free list + refcounts over ``num_blocks`` physical blocks of
    ``block_size`` tokens (16 by default; Habr article §4, "Choosing the block
    size": larger blocks shrink the table, smaller ones waste fewer slots).

    ``free_order`` fixes the order in which free blocks are handed out (a
    seeded permutation gives the scattered placement the pages describe as
    normal); freed blocks go to the back of the queue.
    """

    def __init__(self, num_blocks: int, free_order: Optional[Iterable[int]] = None,
                 block_size: int = BLOCK_SIZE):
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = block_size
        order = list(range(self.num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self._free = deque(order)
        self.ref_count = np.zeros(self.num_blocks, dtype=np.int64)
        self._seqs: dict[int, _Sequence] = {}
        self._next_id = 0

    # ---------------------------------------------------------------- alloc
    def _pop_free(self) -> int:
        if not self._free:
            raise OutOfBlocks("no free KV blocks left")
        b = self._free.popleft()
        self.ref_count[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref_count[b] -= 1
        if self.ref_count[b] == 0:
            self._free.append(b)

    def new_sequence(self, num_tokens: int = 0) -> int:
        """Create a sequence holding ``num_tokens`` tokens (e.g. a prefilled prompt)."""
        sid = self._next_id
        self._next_id += 1
        self._seqs[sid] = _Sequence()
        self.extend(sid, num_tokens)
        return sid

    def extend(self, sid: int, num_tokens: int) -> None:
        """Grow a sequence by ``num_tokens`` tokens, opening blocks as needed.

        Same rules as ``append_slot`` applied token by token, done per block.
        """
        if num_tokens <= 0:
            return
        seq = self._seqs[sid]
        if seq.num_tokens % self.block_size and self.ref_count[seq.blocks[-1]] != 1:
            last = seq.blocks[-1]
            raise SharedBlockWrite(
                f"block {last} is shared by {self.ref_count[last]} sequences; "
                "copy it before writing")
        total = seq.num_tokens + int(num_tokens)
        need = (total + self.block_size - 1) // self.block_size - len(seq.blocks)
        if need > len(self._free):
            raise OutOfBlocks(f"need {need} blocks, {len(self._free)} free")
        for _ in range(need):
            seq.blocks.append(self._pop_free())
        seq.num_tokens = total

    def append_slot(self, sid: int) -> int:
        """Reserve the slot of the sequence's next token and return it.

        A full last block (or none) opens a fresh block; a partially filled
        last block receives the token at its next offset, which requires the
        block to be private to this sequence (see ``append_slot_cow``).
        """
        seq = self._seqs[sid]
        off = seq.num_tokens % self.block_size
        if off == 0:
            seq.blocks.append(self._pop_free())
        else:
            last = seq.blocks[-1]
            if self.ref_count[last] != 1:
                raise SharedBlockWrite(
                    f"block {last} is shared by {self.ref_count[last]} sequences; "
                    "copy it before writing")
        slot = seq.blocks[-1] * self.block_size + off
        seq.num_tokens += 1
        return slot

    def fork(self, parent: int, num_tokens: Optional[int] = None) -> int:
        """New sequence sharing the first ``num_tokens`` tokens of ``parent``.

        The shared blocks gain one reference each; no KV data moves.  If the
        shared length ends inside a block, that partial block is shared too
        and the next token appended to either sequence raises
        ``SharedBlockWrite`` until a copy is made.
        """
        p = self._seqs[parent]
        n = p.num_tokens if num_tokens is None else int(num_tokens)
        if n > p.num_tokens:
            raise ValueError("cannot share more tokens than the parent holds")
        nblk = (n + self.block_size - 1) // self.block_size
        sid = self._next_id
        self._next_id += 1
        child = _Sequence(blocks=list(p.blocks[:nblk]), num_tokens=n)
        for b in child.blocks:
            self.ref_count[b] += 1
        self._seqs[sid] = child
        return sid

    def copy_on_write(self, sid: int, logical_block: Optional[int] = None) -> Optional[Tuple[int, int]]:
        """Give the sequence a private copy of one of its blocks if it is shared.

        Habr article §4, "Copy-on-Write for parallel sampling": a sequence
        that must modify a block other sequences reference copies it first;
        the original stays untouched for the others.  ``logical_block``
        defaults to the last block (where the next token goes; §8 names the
        other case, a speculative correction inside an earlier shared block).

        A private block needs no copy: returns None.  Otherwise a fresh block
        replaces the shared one in this sequence's table, the shared block
        loses this sequence's reference, and ``(src, dst)`` is returned for
        the device copy (``pkv_copy_blocks``), which must run before the
        sequence's next write.
        """
        seq = self._seqs[sid]
        if not seq.blocks:
            return None
        j = len(seq.blocks) - 1 if logical_block is None else int(logical_block)
        if not 0 <= j < len(seq.blocks):
            raise IndexError(f"sequence {sid} has no logical block {j}")
        old = seq.blocks[j]
        if self.ref_count[old] == 1:
            return None
        new = self._pop_free()
        self.ref_count[old] -= 1   # others still hold it: never reaches zero here
        seq.blocks[j] = new
        return old, new

    def append_slot_cow(self, sid: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """``append_slot`` after a copy-on-write of a shared partial last block.

        Returns ``(slot, copy)`` where ``copy`` is the ``(src, dst)`` block pair
        to copy on the device before the token is written, or None.
        """
        seq = self._seqs[sid]
        copy = self.copy_on_write(sid) if seq.num_tokens % self.block_size else None
        return self.append_slot(sid), copy

    def free_sequence(self, sid: int) -> None:
        """Drop a sequence; blocks nobody references any more become free."""
        seq = self._seqs.pop(sid)
        for b in seq.blocks:
            self._release(b)

    # ------------------------------------------------------------ queries
    def blocks(self, sid: int) -> List[int]:
        return list(self._seqs[sid].blocks)

    def num_tokens(self, sid: int) -> int:
        return self._seqs[sid].num_tokens

    def num_free_blocks(self) -> int:
        return len(self._free)

    def blocks_in_use(self) -> int:
        """Distinct physical blocks referenced by at least one sequence."""
        return int(np.count_nonzero(self.ref_count))

    def allocated_slots(self, sid: int) -> int:
        return len(self._seqs[sid].blocks) * self.block_size

    def wasted_slots(self, sid: int) -> int:
        """Reserved but unused slots of one sequence (the tail of its last block)."""
        return self.allocated_slots(sid) - self._seqs[sid].num_tokens

    def block_table(self, seq_ids: Iterable[int], max_blocks: Optional[int] = None,
                    pad: int = -1) -> np.ndarray:
        """int32 table ``[len(seq_ids), max_blocks]``; unused entries hold ``pad``."""
        ids = list(seq_ids)
        need = max((len(self._seqs[s].blocks) for s in ids), default=0)
        width = need if max_blocks is None else int(max_blocks)
        if width < need:
            raise ValueError(f"max_blocks={width} < {need} blocks needed")
        table = np.full((len(ids), max(width, 1)), pad, dtype=np.int32)
        for r, s in enumerate(ids):
            blk = self._seqs[s].blocks
            table[r, :len(blk)] = blk
        return table

    def context_lens(self, seq_ids: Iterable[int]) -> np.ndarray:
        return np.array([self._seqs[s].num_tokens for s in seq_ids], dtype=np.int32)
