"""Helpers that hand a seeded workload to the CPU oracle as plain host arrays."""

from __future__ import annotations

import numpy as np

from paged_kv_cache_23_amd.workloads import Workload, storage_numpy


def oracle_args(wl: Workload, after_append: bool = False, k_pool=None, v_pool=None):
    """Keyword arguments of ``oracle_decode`` for this workload's decode step."""
    tables = wl.block_tables_after if after_append else wl.block_tables
    lens = wl.context_lens_after if after_append else wl.context_lens
    return dict(
        q=storage_numpy(wl.q), q_dtype=wl.q_dtype,
        k_pool=storage_numpy(wl.k_pool) if k_pool is None else k_pool,
        v_pool=storage_numpy(wl.v_pool) if v_pool is None else v_pool,
        kv_dtype=wl.kv_dtype,
        block_tables=tables.numpy(), context_lens=lens.numpy(), scale=wl.scale,
        k_scale=None if wl.k_scale is None else wl.k_scale.numpy(),
        v_scale=None if wl.v_scale is None else wl.v_scale.numpy(),
    )


def oracle_append_args(wl: Workload):
    return dict(
        k_pool=storage_numpy(wl.k_pool), v_pool=storage_numpy(wl.v_pool),
        k_new=storage_numpy(wl.k_new), v_new=storage_numpy(wl.v_new),
        slot_mapping=wl.slot_mapping.numpy(), kv_dtype=wl.kv_dtype,
        k_scale=None if wl.k_scale is None else wl.k_scale.numpy(),
        v_scale=None if wl.v_scale is None else wl.v_scale.numpy(),
    )


def f32_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)
