"""GPU parity of pkv_paged_decode_shared (decode over a batch that shares
its leading blocks: the prefix read once for all sequences) against the fp64
oracle's decode over each sequence's own table, through the C ABI."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

from paged_kv_cache_23_amd import ops
from paged_kv_cache_23_amd import workloads as W
from paged_kv_cache_23_amd.workloads import build_workload
from tests.gpu_util import Dev, assert_close, oracle_full

pytestmark = pytest.mark.gpu


def _shared(dev: Dev, prefix_tokens: int, max_context_len=None, workers=0, workspace=None):
    wl = dev.wl
    mctx = int(wl.context_lens.max()) if max_context_len is None else max_context_len
    return ops.paged_decode_shared(dev.q, dev.k_pool, dev.v_pool, dev.tables, dev.lens, wl.scale, prefix_tokens,
                                   k_scale=dev.k_scale, v_scale=dev.v_scale, max_context_len=mctx,
                                   num_workers=workers, workspace=workspace)


def _one_launch_workers() -> int:
    """One tail wave per SIMD: with a bf16 or fp8 cache the call then runs the
    tail walk and the prefix part in one launch."""
    return 4 * torch.cuda.get_device_properties(0).multi_processor_count


def _tails(rng, B, hi):
    """Tail lengths after the prefix: empty, 1, one chunk's edges, the rest random."""
    fixed = [0, 1, 31, 32, 33, 100]
    return [fixed[b] if b < len(fixed) else int(rng.integers(0, hi)) for b in range(B)]


# (query heads per kv head) x batch = columns of the prefix pass: under one
# MFMA tile (8), one workgroup, several with a ragged last one (528, 1200).
@pytest.mark.parametrize("kv_dtype,D,G,B,P,bs", [
    ("bf16", 128, 4, 37, 640, 16), ("bf16", 64, 16, 33, 1024, 16), ("bf16", 128, 1, 300, 4096, 256),
    ("bf16", 128, 8, 1, 320, 16), ("fp8", 128, 8, 20, 2000, 16), ("fp8", 64, 2, 9, 512, 32),
    ("f32", 64, 2, 9, 256, 16), ("f32", 128, 4, 70, 1024, 64),
    # long prefixes: 128 key segments whose partial accumulators (bf16 for
    # bf16 and fp8 caches) the merge combines
    ("bf16", 128, 4, 8, 16384, 16), ("fp8", 128, 4, 6, 16384, 16), ("f32", 64, 2, 4, 8192, 16),
    # prefixes that end half way into a 32-token chunk (1040 = 32.5 chunks)
    ("bf16", 128, 4, 24, 1040, 16), ("bf16", 64, 8, 40, 528, 16),
])
@pytest.mark.parametrize("one_launch", [False, True])
def test_shared_parity(kv_dtype, D, G, B, P, bs, one_launch):
    rng = np.random.default_rng(B * 7 + P)
    lens = [P + t for t in _tails(rng, B, 300)]
    wl = build_workload("shared", lens, 2 * G, 2, D, kv_dtype, seed=B + P, shared_prefix=P, rng=rng,
                        block_size=bs)
    workers = _one_launch_workers() if one_launch else 0
    print(f"shared {kv_dtype} D={D} G={G} B={B} P={P} bs={bs} workers={workers}", flush=True)
    out = _shared(Dev(wl), P, workers=workers)
    assert out.shape == wl.q.shape
    assert_close(out, oracle_full(wl), kv_dtype)


def test_any_block_aligned_part_of_the_shared_prefix():
    """prefix_tokens may name any whole-block part of what the rows share
    (0 runs the plain decode); the result is the same decode every time."""
    rng = np.random.default_rng(5)
    P = 800
    wl = build_workload("shared", [P + t for t in _tails(rng, 24, 200)], 16, 4, 128, "bf16", seed=5,
                        shared_prefix=P, rng=rng)
    dev = Dev(wl)
    ref = oracle_full(wl)
    for p in (0, 16, 400, 784, 800):
        assert_close(_shared(dev, p), ref, "bf16")
        assert_close(_shared(dev, p, workers=_one_launch_workers()), ref, "bf16")


def test_every_tail_empty():
    """Every sequence is exactly the prefix: the output comes from the prefix
    pass alone."""
    P = 1024
    wl = build_workload("shared", [P] * 12, 32, 8, 128, "bf16", seed=6, shared_prefix=P)
    dev = Dev(wl)
    ref = oracle_full(wl)
    assert_close(_shared(dev, P), ref, "bf16")
    assert_close(_shared(dev, P, workers=_one_launch_workers()), ref, "bf16")


@pytest.mark.parametrize("scale", [-0.07, 0.0])
def test_scale_signs(scale):
    """A negative score scale (the prefix part flips the queries' signs
    instead) and a zero one (every visible token weighs the same), on both
    paths."""
    rng = np.random.default_rng(12)
    P = 528
    wl = build_workload("shared", [P + t for t in _tails(rng, 30, 200)], 32, 8, 128, "bf16", seed=12,
                        shared_prefix=P, rng=rng)
    wl = dataclasses.replace(wl, scale=scale)
    dev = Dev(wl)
    ref = oracle_full(wl)
    for workers in (0, _one_launch_workers()):
        assert_close(_shared(dev, P, workers=workers), ref, "bf16")


def test_worker_counts_and_a_reused_workspace():
    rng = np.random.default_rng(7)
    P = 512
    wl = build_workload("shared", [P + t for t in _tails(rng, 40, 600)], 32, 8, 128, "bf16", seed=7,
                        shared_prefix=P, rng=rng)
    dev = Dev(wl)
    ref = oracle_full(wl)
    mctx = int(wl.context_lens.max())
    full = _one_launch_workers()
    counts = (4, 64, 1024, full, 4)
    need = max(ops.shared_decode_workspace_bytes(dev.k_pool, dev.v_pool, 32, 40, mctx, P, w) for w in counts)
    ws = ops.new_workspace(need, dev.q.device)
    for w in counts:             # partials of the earlier calls stay behind
        for p in (P, 0):         # the plain decode (no prefix) shares the workspace too
            assert_close(_shared(dev, p, workers=w, workspace=ws), ref, "bf16")


def test_lengths_clamped_by_max_context_len():
    rng = np.random.default_rng(8)
    P = 320
    wl = build_workload("shared", [P + t for t in _tails(rng, 16, 400)], 32, 8, 128, "bf16", seed=8,
                        shared_prefix=P, rng=rng)
    bound = P + 40
    out = _shared(Dev(wl), P, max_context_len=bound)
    clamped = dataclasses.replace(wl, context_lens=wl.context_lens.clamp(max=bound))
    assert_close(out, oracle_full(clamped), "bf16")


def test_argument_errors():
    P = 320
    wl = build_workload("shared", [P + 5, P + 60], 8, 2, 128, "bf16", seed=9, shared_prefix=P)
    dev = Dev(wl)
    with pytest.raises(RuntimeError, match="invalid"):
        _shared(dev, P - 8)                               # not a whole number of blocks
    with pytest.raises(RuntimeError, match="invalid"):
        _shared(dev, P, max_context_len=P - 16)           # longer than the bound on the lengths
    with pytest.raises(RuntimeError, match="invalid"):
        _shared(dev, 16 * (wl.block_tables.shape[1] + 1), max_context_len=10 ** 6)   # past the table


# ---------------------------------------------------------------------------
# Full-size batches, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------
def test_shared_prefix_256_all_outputs():
    """256 sequences over one 4096-token prefix (+ 64..512-token tails): every
    output of the shared-prefix call against the oracle."""
    wl = W.shared_prefix_256()
    print("shared-prefix-256 through the shared-prefix call", flush=True)
    dev = Dev(wl)
    ref = oracle_full(wl)
    full = _one_launch_workers()
    # the default (one launch: the tails give every SIMD a wave), then the
    # three-launch path (one tail wave fewer per workgroup's worth)
    for workers in (0, full - 4):
        err = assert_close(_shared(dev, 4096, workers=workers), ref, "bf16")
        print(f"shared-prefix-256 (shared call, workers={workers}) max|err| = {err:.3g}")


def test_best_of_8_all_outputs():
    """Best-of-8 over a 2,000-token prompt (125 shared blocks), with the
    library's worker count and in one launch."""
    wl = W.best_of_8()
    dev = Dev(wl)
    ref = oracle_full(wl)
    for workers in (0, _one_launch_workers()):
        err = assert_close(_shared(dev, 2000, workers=workers), ref, "bf16")
        print(f"best-of-8 (shared call, workers={workers}) max|err| = {err:.3g}")


def test_policy_picks_either_path_with_the_same_result():
    """always=False consults the crossover: a best-of-8 batch runs the plain
    decode, 64 sequences over a 4,096-token prefix the cascade; both agree
    with the oracle."""
    for B, P in ((8, 2000), (64, 4096)):
        rng = np.random.default_rng(B)
        wl = build_workload("shared", [P + int(t) for t in rng.integers(1, 201, size=B)], 32, 8, 128, "bf16",
                            seed=B, shared_prefix=P, rng=rng)
        dev = Dev(wl)
        assert ops.shared_prefix_pays(dev.k_pool, dev.v_pool, 32, B, P) == (B == 64)
        out = ops.paged_decode_shared(dev.q, dev.k_pool, dev.v_pool, dev.tables, dev.lens, wl.scale, P,
                                      max_context_len=int(wl.context_lens.max()), always=False)
        assert_close(out, oracle_full(wl), "bf16")
