"""CPU oracle for paged decode attention over a block-table KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
helpers with the HIP library; the two meet only through arrays that a seeded
input generator (which holds none of the method's arithmetic) produces.

Every function is plain fp64 NumPy that follows the definitions on the
source pages (cited in each docstring) and can be checked against them by eye.
"""

from .paged_attention import (  # noqa: F401
    BLOCK_SIZE,
    bf16_bits_to_f64,
    block_size_of,
    e4m3_decode,
    e4m3_encode,
    gather_slab,
    kv_bytes_per_token,
    oracle_append,
    oracle_attention_multi,
    oracle_copy_blocks,
    oracle_decode,
    oracle_decode_pairs,
    softmax_weights,
)
