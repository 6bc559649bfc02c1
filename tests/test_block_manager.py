"""Pins of the host block manager against the pages' worked examples and rules."""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

from paged_kv_cache_23_amd import BlockManager, OutOfBlocks, SharedBlockWrite

G = os.path.join(os.path.dirname(__file__), "golden")
WORKED = json.load(open(os.path.join(G, "paging_worked_example.json")))
BO8 = json.load(open(os.path.join(G, "best_of_8.json")))


def test_worked_example_1024_plus_10():
    """Habr article §4 step-by-step example: 64 prefill blocks, token 1025 opens
    block 64 at its first slot, 65 blocks / 1040 slots / 6 wasted (0.6%)."""
    w = WORKED
    prefix = w["table_prefix"]
    rest = [b for b in range(1024) if b not in prefix]
    bm = BlockManager(1024, free_order=prefix + rest)
    s = bm.new_sequence(w["prompt_tokens"])
    assert len(bm.blocks(s)) == w["prefill_blocks"]
    assert bm.blocks(s)[:3] == prefix
    slot = bm.append_slot(s)                      # token 1025
    blocks = bm.blocks(s)
    assert len(blocks) - 1 == w["token_1025"]["logical_block"]
    assert slot == blocks[64] * 16 + (w["token_1025"]["slot_one_based"] - 1)
    bm.extend(s, w["generated_tokens"] - 1)
    assert bm.num_tokens(s) == w["used_tokens"]
    assert bm.num_tokens(s) - 64 * 16 == w["after_generation_last_block_used"]
    assert len(bm.blocks(s)) == w["allocated_blocks"]
    assert bm.allocated_slots(s) == w["allocated_slots"]
    assert bm.wasted_slots(s) == w["wasted_slots"]
    assert round(100 * bm.wasted_slots(s) / bm.allocated_slots(s), 1) == w["wasted_percent_printed"]
    naive_waste = w["naive_max_seq_len"] - w["used_tokens"]
    assert naive_waste == w["naive_wasted_slots"]
    assert round(100 * naive_waste / w["naive_max_seq_len"], 1) == w["naive_wasted_percent_printed"]


@pytest.mark.parametrize("n", list(range(0, 70)) + [1023, 1024, 1025, 4097])
def test_waste_at_most_one_partial_block(n):
    bm = BlockManager(300)
    s = bm.new_sequence(n)
    assert 0 <= bm.wasted_slots(s) <= WORKED["max_waste_per_sequence_tokens"]
    assert len(bm.blocks(s)) == -(-n // 16)


def test_slots_follow_append_order_and_open_blocks():
    rng = np.random.default_rng(0)
    bm = BlockManager(64, free_order=rng.permutation(64))
    s = bm.new_sequence(0)
    slots = [bm.append_slot(s) for _ in range(50)]
    blocks = bm.blocks(s)
    assert slots == [blocks[t // 16] * 16 + t % 16 for t in range(50)]
    assert len(set(slots)) == 50


def test_best_of_8_accounting():
    """Chapter 8 §8.1: best-of-8 on a 2000-token prompt, 16,800 -> 2,800 token
    slots with 100-token tails; the prompt is 125 blocks (Habr article §7)."""
    b = BO8
    tail = b["tail_tokens_reading"]
    # unshared: eight independent copies
    bm = BlockManager(2000)
    ids = [bm.new_sequence(b["prompt_tokens"] + tail) for _ in range(b["samples"])]
    unshared_tokens = sum(bm.num_tokens(s) for s in ids)
    unshared_blocks = bm.blocks_in_use()
    # shared: one refcounted prompt, eight private tails
    bm2 = BlockManager(2000)
    root = bm2.new_sequence(b["prompt_tokens"])
    assert len(bm2.blocks(root)) == b["prompt_blocks"]
    kids = []
    for _ in range(b["samples"]):
        k = bm2.fork(root)
        bm2.extend(k, tail)
        kids.append(k)
    bm2.free_sequence(root)
    shared_tokens = b["prompt_tokens"] + sum(bm2.num_tokens(k) - b["prompt_tokens"] for k in kids)
    assert unshared_tokens == b["printed_unshared"]
    assert shared_tokens == b["printed_shared"]
    assert unshared_blocks == 1056 and bm2.blocks_in_use() == 181
    assert all(bm2.ref_count[blk] == b["samples"] for blk in bm2.blocks(kids[0])[:125])


def test_refcounts_and_free_on_release():
    bm = BlockManager(10)
    root = bm.new_sequence(32)          # 2 blocks
    a = bm.fork(root)
    bm.extend(a, 5)
    assert [bm.ref_count[x] for x in bm.blocks(root)] == [2, 2]
    bm.free_sequence(root)
    assert [bm.ref_count[x] for x in bm.blocks(a)] == [1, 1, 1]
    free_before = bm.num_free_blocks()
    bm.free_sequence(a)
    assert bm.num_free_blocks() == free_before + 3
    assert bm.blocks_in_use() == 0


def test_write_into_shared_partial_block_is_refused():
    bm = BlockManager(10)
    root = bm.new_sequence(20)          # partial second block
    child = bm.fork(root)
    with pytest.raises(SharedBlockWrite):
        bm.append_slot(child)
    with pytest.raises(SharedBlockWrite):
        bm.extend(root, 1)
    # a prefix that ends on a block boundary leaves appends free to go
    root2 = bm.new_sequence(16)
    c2 = bm.fork(root2)
    bm.append_slot(c2)
    bm.append_slot(root2)
    assert bm.blocks(c2)[1] != bm.blocks(root2)[1]


def test_out_of_blocks():
    bm = BlockManager(2)
    bm.new_sequence(32)
    with pytest.raises(OutOfBlocks):
        bm.new_sequence(1)


def test_block_table_padding():
    bm = BlockManager(8, free_order=[3, 1, 4, 0, 5, 2, 6, 7])
    a = bm.new_sequence(17)
    b = bm.new_sequence(1)
    t = bm.block_table([a, b], 4)
    assert t.dtype == np.int32 and t.shape == (2, 4)
    assert t.tolist() == [[3, 1, -1, -1], [4, -1, -1, -1]]
    assert bm.context_lens([a, b]).tolist() == [17, 1]


def test_copy_on_write_gives_a_private_block():
    """Habr article §4, "Copy-on-Write for parallel sampling": the sequence that
    writes gets a fresh copy of the shared block; the other keeps the original;
    reference counts follow and both can then append."""
    bm = BlockManager(10)
    root = bm.new_sequence(20)               # blocks [0, 1]; block 1 holds 4 tokens
    child = bm.fork(root)
    assert bm.ref_count[1] == 2
    assert bm.copy_on_write(child) == (1, 2)
    assert bm.blocks(child) == [0, 2] and bm.blocks(root) == [0, 1]
    assert (bm.ref_count[0], bm.ref_count[1], bm.ref_count[2]) == (2, 1, 1)
    assert bm.copy_on_write(child) is None and bm.copy_on_write(root) is None   # both private now
    assert bm.append_slot(child) == 2 * 16 + 4
    assert bm.append_slot(root) == 1 * 16 + 4
    # an earlier, full shared block (Habr §8: a speculative correction inside it)
    src, dst = bm.copy_on_write(child, 0)
    assert src == 0 and bm.blocks(child)[0] == dst and bm.ref_count[0] == 1
    # the combined call: root now holds 21 tokens
    c2 = bm.fork(root)
    slot, copy = bm.append_slot_cow(c2)
    assert copy == (1, bm.blocks(c2)[1]) and slot == bm.blocks(c2)[1] * 16 + 5
    assert bm.append_slot_cow(c2)[1] is None  # private already
    # freeing the copies returns them; the original lives on with the root
    used = bm.blocks_in_use()
    bm.free_sequence(c2)
    assert bm.blocks_in_use() == used - 1 and bm.ref_count[1] == 1


@pytest.mark.parametrize("bs,worst", [(16, 15), (256, 255)])
def test_block_size_bounds_the_waste(bs, worst):
    """Habr §4 "Choosing the block size": 16-token blocks waste at most 15
    slots per request, 256-token blocks up to 255."""
    bm = BlockManager(4096, block_size=bs)
    wastes = []
    for n in range(1, 3 * bs + 2):
        s = bm.new_sequence(n)
        wastes.append(bm.wasted_slots(s))
        assert bm.allocated_slots(s) == -(-n // bs) * bs
        bm.free_sequence(s)
    assert max(wastes) == worst and min(wastes) == 0
