"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The compute lives in ``libpkv.so`` (HIP kernels behind a C ABI declared in
``include/pkv.h``); ``paged_kv_cache_23_amd.ops`` is a thin ctypes binding
with the same entry-point names.  Importing the package loads nothing: the
library is opened on the first call, and a missing library is an error.
"""

from .block_manager import BlockManager, OutOfBlocks, SharedBlockWrite  # noqa: F401

__all__ = ["BlockManager", "OutOfBlocks", "SharedBlockWrite"]
