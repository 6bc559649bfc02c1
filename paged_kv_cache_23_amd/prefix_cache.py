"""ctypes binding of the host block pool with a prefix-cache index
(``pkv_pool_*`` in ``include/pkv.h``): argument marshalling only; the pool,
the hash chain and the LRU queue live in the library's C++ code."""

from __future__ import annotations

import ctypes
from typing import List, Sequence

import numpy as np

from . import ops

ENOSPACE = -5

_bound = False


def _lib() -> ctypes.CDLL:
    global _bound
    lib = ops.library()
    if not _bound:
        P, I32, I64, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        sigs = {
            "pkv_pool_create": (P, [I32, I32]),
            "pkv_pool_destroy": (None, [P]),
            "pkv_pool_match_prefix": (I32, [P, P, I32, U64, P, I32]),
            "pkv_pool_allocate": (I32, [P, I32, P]),
            "pkv_pool_cache_blocks": (I32, [P, P, I32, U64, P, I32]),
            "pkv_pool_free": (ctypes.c_int, [P, P, I32]),
            "pkv_pool_ref": (ctypes.c_int, [P, P, I32]),
            "pkv_pool_block_hash": (ctypes.c_int, [P, P, I32, U64, P, I32]),
            "pkv_pool_num_free": (I32, [P]),
            "pkv_pool_num_cached": (I32, [P]),
            "pkv_pool_ref_count": (I32, [P, I32]),
            "pkv_pool_evictions": (I64, [P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _bound = True
    return lib


def _i32(xs: Sequence[int]) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(xs, dtype=np.int32))


class PrefixCachePool:
    """Blocks of ``block_size`` tokens with reference counts, an LRU queue of
    unreferenced blocks and a hash-chain index of full blocks."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        self._lib = _lib()
        self._h = self._lib.pkv_pool_create(int(num_blocks), int(block_size))
        if not self._h:
            raise ValueError("pkv_pool_create failed (bad sizes or out of memory)")
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def close(self) -> None:
        if self._h:
            self._lib.pkv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def _check(self, st: int, what: str) -> int:
        if st < 0:
            raise RuntimeError(f"{what}: {self._lib.pkv_strerror(st).decode()} (status {st})")
        return st

    def match_prefix(self, tokens: Sequence[int], extra_key: int = 0) -> List[int]:
        """Cached blocks covering the request's longest cached prefix (each gains a reference)."""
        t = _i32(tokens)
        cap = max(len(t) // self.block_size, 1)
        out = np.empty(cap, dtype=np.int32)
        n = self._check(self._lib.pkv_pool_match_prefix(self._h, t.ctypes.data, len(t), extra_key,
                                                        out.ctypes.data, cap), "match_prefix")
        return out[:n].tolist()

    def allocate(self, count: int) -> List[int]:
        out = np.empty(max(count, 1), dtype=np.int32)
        st = self._lib.pkv_pool_allocate(self._h, int(count), out.ctypes.data)
        if st == ENOSPACE:
            raise MemoryError(f"{count} blocks requested, {self.num_free} free")
        self._check(st, "allocate")
        return out[:count].tolist()

    def cache_blocks(self, tokens: Sequence[int], blocks: Sequence[int], extra_key: int = 0) -> int:
        t, b = _i32(tokens), _i32(blocks)
        return self._check(self._lib.pkv_pool_cache_blocks(self._h, t.ctypes.data, len(t), extra_key,
                                                           b.ctypes.data, len(b)), "cache_blocks")

    def free(self, blocks: Sequence[int]) -> None:
        b = _i32(blocks)
        self._check(self._lib.pkv_pool_free(self._h, b.ctypes.data, len(b)), "free")

    def ref(self, blocks: Sequence[int]) -> None:
        """One more reference to each block (another sequence shares it)."""
        b = _i32(blocks)
        self._check(self._lib.pkv_pool_ref(self._h, b.ctypes.data, len(b)), "ref")

    def block_hashes(self, tokens: Sequence[int], extra_key: int = 0) -> List[bytes]:
        t = _i32(tokens)
        cap = len(t) // self.block_size
        out = np.zeros(max(cap, 1) * 32, dtype=np.uint8)
        n = self._check(self._lib.pkv_pool_block_hash(self._h, t.ctypes.data, len(t), extra_key,
                                                      out.ctypes.data, cap), "block_hash")
        return [out[32 * j:32 * (j + 1)].tobytes() for j in range(n)]

    def admit(self, tokens: Sequence[int], extra_key: int = 0):
        """A new request: reuse its cached prefix and allocate the rest.
        Returns (blocks for every token, number of hit blocks)."""
        hit = self.match_prefix(tokens, extra_key)
        need = -(-len(tokens) // self.block_size) - len(hit)
        try:
            fresh = self.allocate(need)
        except MemoryError:
            self.free(hit)
            raise
        return hit + fresh, len(hit)

    @property
    def num_free(self) -> int:
        return self._lib.pkv_pool_num_free(self._h)

    @property
    def num_cached(self) -> int:
        return self._lib.pkv_pool_num_cached(self._h)

    @property
    def evictions(self) -> int:
        return self._lib.pkv_pool_evictions(self._h)

    def ref_count(self, block: int) -> int:
        return self._check(self._lib.pkv_pool_ref_count(self._h, int(block)), "ref_count")


class CachingBlockManager:
    """Sequences over a ``PrefixCachePool``: the pool (C++) is the single owner
    of every block's reference count, of the LRU queue of unreferenced blocks
    and of the hash index; this class keeps only each sequence's token ids
    and block list, and hands out the block tables, lengths and slots the
    kernels take.

    Habr KV-Cache article, section 7 "That same Cache Read": a request first
    reuses the blocks of its longest cached prefix (each gains a reference)
    and computes only the rest; full blocks are indexed once their K/V are
    written and are never modified afterwards.  Section 4: a fresh block is
    opened when the last one is full; a fork shares blocks by reference
    (parallel sampling), and a write into a shared partial block needs a
    copy first (copy-on-write).  Slots are ``block * block_size + offset``.
    """

    def __init__(self, pool: PrefixCachePool, extra_key: int = 0):
        self.pool = pool
        self.block_size = pool.block_size
        self.extra_key = int(extra_key)
        self._tokens: dict = {}
        self._blocks: dict = {}
        self._next = 0

    def admit(self, tokens: Sequence[int]):
        """A new request of ``tokens``: reuse its cached prefix, allocate blocks
        for the rest.  Returns (sequence id, tokens whose K/V are already
        cached); the caller writes the K/V of the tokens after those."""
        blocks, hit = self.pool.admit(tokens, self.extra_key)
        sid = self._next
        self._next += 1
        self._tokens[sid] = [int(t) for t in tokens]
        self._blocks[sid] = list(blocks)
        return sid, hit * self.block_size

    def mark_computed(self, sid: int) -> int:
        """The sequence's K/V are written: index its full blocks (returns how
        many were newly indexed)."""
        return self.pool.cache_blocks(self._tokens[sid], self._blocks[sid], self.extra_key)

    def slots(self, sid: int, start: int, end: int) -> np.ndarray:
        """int64 slots of token positions [start, end) of the sequence."""
        pos = np.arange(start, end, dtype=np.int64)
        blk = np.asarray(self._blocks[sid], dtype=np.int64)[pos // self.block_size]
        return blk * self.block_size + pos % self.block_size

    def append_slot(self, sid: int, token: int) -> int:
        """Reserve the slot of the sequence's next token (id ``token``); a full
        last block opens a fresh one, a shared partial one is refused (copy it
        first with ``copy_on_write``).  A block that becomes full is indexed
        when ``mark_computed`` runs after its K/V are written."""
        from .block_manager import SharedBlockWrite

        toks, blks = self._tokens[sid], self._blocks[sid]
        off = len(toks) % self.block_size
        if off == 0:
            blks.extend(self.pool.allocate(1))
        elif self.pool.ref_count(blks[-1]) != 1:
            raise SharedBlockWrite(f"block {blks[-1]} is shared; copy it before writing")
        toks.append(int(token))
        return blks[-1] * self.block_size + off

    def fork(self, sid: int) -> int:
        """A new sequence sharing all of ``sid``'s tokens and blocks."""
        self.pool.ref(self._blocks[sid])
        new = self._next
        self._next += 1
        self._tokens[new] = list(self._tokens[sid])
        self._blocks[new] = list(self._blocks[sid])
        return new

    def copy_on_write(self, sid: int):
        """A private copy of the sequence's last block if others share it:
        returns (src, dst) for ``pkv_copy_blocks`` (to run before the next
        write), or None when the block is private."""
        blks = self._blocks[sid]
        if not blks or self.pool.ref_count(blks[-1]) == 1:
            return None
        dst = self.pool.allocate(1)[0]
        src = blks[-1]
        self.pool.free([src])          # this sequence's reference; others keep theirs
        blks[-1] = dst
        return src, dst

    def free_sequence(self, sid: int) -> None:
        """The request finished: its blocks lose a reference (unreferenced ones
        stay indexed in the LRU queue until reused)."""
        self.pool.free(self._blocks.pop(sid))
        del self._tokens[sid]

    def blocks(self, sid: int) -> List[int]:
        return list(self._blocks[sid])

    def num_tokens(self, sid: int) -> int:
        return len(self._tokens[sid])

    def block_table(self, sids: Sequence[int], max_blocks: int = 0, pad: int = -1) -> np.ndarray:
        rows = [self._blocks[s] for s in sids]
        width = max(max((len(r) for r in rows), default=0), int(max_blocks), 1)
        table = np.full((len(rows), width), pad, dtype=np.int32)
        for i, r in enumerate(rows):
            table[i, :len(r)] = r
        return table

    def context_lens(self, sids: Sequence[int]) -> np.ndarray:
        return np.array([len(self._tokens[s]) for s in sids], dtype=np.int32)
