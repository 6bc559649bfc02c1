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
