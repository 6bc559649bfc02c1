"""Host-side helpers of bench.py: the shared leading blocks of a batch and the
distinct KV bytes a decode reads (no GPU)."""

from __future__ import annotations

import numpy as np

import bench
from paged_kv_cache_23_amd import workloads as W
from paged_kv_cache_23_amd.workloads import build_workload


def test_common_prefix_of_best_of_8():
    wl = W.best_of_8()
    assert bench.common_prefix_tokens(wl.block_tables.numpy(), wl.context_lens.numpy(), 16) == 2000


def test_common_prefix_stops_at_the_first_difference_and_the_shortest_sequence():
    t = np.array([[5, 6, 7, 8], [5, 6, 9, 10], [5, 6, 7, 11]])
    assert bench.common_prefix_tokens(t, np.array([64, 64, 64]), 16) == 32
    assert bench.common_prefix_tokens(t, np.array([64, 20, 64]), 16) == 16   # one holds a single full block
    assert bench.common_prefix_tokens(t[:1], np.array([50]), 16) == 48        # one row shares its full blocks
    assert bench.common_prefix_tokens(np.zeros((0, 4), np.int32), np.zeros(0, np.int32), 16) == 0


def test_unique_bytes_count_the_prefix_once():
    P, tails = 512, [16, 40, 0]
    wl = build_workload("s", [P + t for t in tails], 8, 2, 64, "bf16", seed=3, shared_prefix=P)
    per_token = 2 * 2 * 64 * 2   # K and V, 2 kv heads, head_dim 64, bf16
    assert bench.unique_kv_bytes(wl, False) == (P + sum(tails)) * per_token
    assert wl.kv_bytes() == (3 * P + sum(tails)) * per_token


def test_committed_traffic_profiles_are_well_formed():
    """Every committed HBM-counter summary that a bench line reports as its
    roofline `traffic` records the source hash it was taken on and its bytes
    per launch, which lie just above the launch unit's algorithmic bytes
    where those are a fixed figure.  (A summary taken on older code is not
    reported by bench.py; the rejection is tested below.)"""
    import os
    import re
    cases = [("paged_decode_llama3-8b-b64", None),
             ("copy_blocks_kernel_copy-4096", 2 * 2 * 4096 * 32768),
             ("prefill_kernel_prefill-70b-10k", None),
             ("paged_decode_shared_shared-prefix-256", 326_193_152),
             ("append_kernel_append-65536-bf16", 65536 * 8 * 128 * 2 * 4),
             ("append_kernel_append-65536-fp8", 65536 * 8 * 128 * 2 * 3)]
    for name, algo in cases:
        text = open(os.path.join(bench.PROFILE_DIR, f"{name}_hbm_traffic.txt")).read()
        assert re.search(r"^source_hash:\s*[0-9a-f]{16}\b", text, re.M), name
        t = float(re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M).group(1))
        assert t > 0, name
        if algo is not None:
            assert algo <= t <= 1.35 * algo, (name, t, algo)


def test_committed_traffic_rejects_a_changed_source(tmp_path, monkeypatch):
    """A summary whose recorded source hash differs from the current code is
    not reported."""
    text = "source_hash: 0123456789abcdef\nhbm_bytes_per_launch: 1000\n"
    (tmp_path / "append_kernel_x_hbm_traffic.txt").write_text(text)
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.committed_traffic("x", "append_kernel", bench.APPEND_SOURCES) is None
    h = bench.kernel_source_hash(bench.APPEND_SOURCES)
    (tmp_path / "append_kernel_x_hbm_traffic.txt").write_text(text.replace("0123456789abcdef", h))
    assert bench.committed_traffic("x", "append_kernel", bench.APPEND_SOURCES) == 1000.0


def test_oracle_pool_gives_the_oracles_results():
    """The bench's oracle leg runs the oracle unchanged on several host
    processes: what they return equals the oracle called directly."""
    import numpy as np

    import bench
    import oracle
    from paged_kv_cache_23_amd.workloads import build_workload, storage_numpy

    wl = build_workload("pool", [5, 40, 100], 8, 2, 64, "fp8", seed=3)
    args = dict(q=storage_numpy(wl.q), k_pool=storage_numpy(wl.k_pool), v_pool=storage_numpy(wl.v_pool),
                tables=wl.block_tables.numpy(), lens=wl.context_lens.numpy(), k_scale=wl.k_scale.numpy(),
                v_scale=wl.v_scale.numpy())
    pool = bench.OraclePool(args, dict(q_dtype="bf16", kv_dtype="fp8", scale=wl.scale), 2)
    try:
        pairs = [(b, g) for b in range(3) for g in range(2)]
        got = np.concatenate(pool.map(bench._oracle_pairs_task, [[p] for p in pairs]))
    finally:
        pool.close()
    ref = oracle.oracle_decode_pairs(args["q"], "bf16", args["k_pool"], args["v_pool"], "fp8", args["tables"],
                                     args["lens"], wl.scale, pairs, args["k_scale"], args["v_scale"])
    assert np.array_equal(got, ref)


def test_cpu_baseline_reports_the_cores_it_used():
    import bench
    from paged_kv_cache_23_amd.workloads import build_workload

    wl = build_workload("cores", [64, 300], 8, 2, 64, "bf16", seed=4)
    res = bench.cpu_baseline(wl, min_seconds=0.2, max_reps=3)
    assert res["cores"] == bench.host_cores() >= 1
    assert res["value"] > 0 and res["kind"] == "oracle"
