"""The chunked-prefill workload (Habr section 6's 10,000-token prompt in
2048-token chunks) and its flop count, on the CPU."""

from __future__ import annotations

import numpy as np

from paged_kv_cache_23_amd.workloads import prefill_chunks


def test_chunks_follow_the_worked_example():
    """Habr section 6: under a 2048-token budget a 10,000-token prompt runs as
    chunks of 2048, 2048, 2048, 2048 and 1808 tokens; chunk k's cache holds
    every token up to the end of chunk k."""
    steps = prefill_chunks(prompt_tokens=10000, chunk=2048, num_q_heads=4, num_kv_heads=1, head_dim=64)
    assert [s.q.shape[1] for s in steps] == [2048, 2048, 2048, 2048, 1808]
    assert [int(s.wl.context_lens[0]) for s in steps] == [2048, 4096, 6144, 8192, 10000]
    # one pool and one table shared by every step: 625 blocks of 16 tokens
    assert all(s.wl.k_pool is steps[0].wl.k_pool for s in steps)
    assert (steps[0].wl.block_tables[0] >= 0).sum() == 625


def test_flops_count_every_causal_pair_once():
    """4 * Hq * D flops per (query, visible key) pair: compare with a brute
    count of the causal pairs of a small chunk."""
    steps = prefill_chunks(prompt_tokens=100, chunk=48, num_q_heads=4, num_kv_heads=2, head_dim=64)
    for s in steps:
        n, L = int(s.wl.context_lens[0]), s.q.shape[1]
        pos = np.arange(n - L, n)
        pairs = sum(int(np.sum(np.arange(n) <= p)) for p in pos)
        assert s.flops() == 4 * 4 * 64 * pairs
    # the whole prompt: every (query, key) pair with key <= query, once
    assert sum(s.flops() for s in steps) == 4 * 4 * 64 * (100 * 101 // 2)
