"""kv_append on the GPU is bit-exact against the oracle, with every byte of
both pools compared (untouched bytes must stay untouched)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_23_amd import ops
from paged_kv_cache_23_amd.workloads import build_workload, fp8_b256, storage_numpy, tiny_fp32
from tests.gpu_util import Dev, host

pytestmark = pytest.mark.gpu


def _check_append(wl):
    dev = Dev(wl)
    dev.append()
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.oracle_append(
        storage_numpy(wl.k_pool), storage_numpy(wl.v_pool), storage_numpy(wl.k_new), storage_numpy(wl.v_new),
        wl.slot_mapping.numpy(), wl.kv_dtype,
        None if wl.k_scale is None else wl.k_scale.numpy(),
        None if wl.v_scale is None else wl.v_scale.numpy())
    got_k, got_v = host(dev.k_pool), host(dev.v_pool)
    assert np.array_equal(got_k.view(np.uint8), ref_k.view(np.uint8))
    assert np.array_equal(got_v.view(np.uint8), ref_v.view(np.uint8))


def test_append_tiny_fp32():
    _check_append(tiny_fp32())


@pytest.mark.parametrize("kv_dtype,D", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128),
                                        ("fp8", 64), ("fp8", 128)])
def test_append_dtypes_and_dims(kv_dtype, D):
    wl = build_workload("append", [0, 15, 16, 17, 31, 100], 8, 4, D, kv_dtype, seed=21, with_append=True)
    _check_append(wl)


def test_append_padding_and_out_of_range_slots_write_nothing():
    wl = build_workload("pad", [3, 40, 16], 4, 2, 128, "bf16", seed=5, with_append=True)
    slots = wl.slot_mapping.clone()
    slots[1] = -1                                   # padding token
    slots[2] = wl.num_blocks * 16 + 7               # past the pool: skipped
    wl.slot_mapping = slots
    _check_append(wl)


def test_append_fp8_step_shape():
    """256 sequences, one appended bf16 token each, quantised into the E4M3 pool."""
    _check_append(fp8_b256())


@pytest.mark.parametrize("scale", [1.0, 0.37, 1.0 / 448.0, 3.5e-3])
def test_fp8_quantiser_exhaustive(scale):
    """Every bf16 input pattern encodes to the same E4M3 code on the GPU and in
    the oracle: one kv head, 512 tokens x 128 dims = all 65,536 patterns."""
    D, Hkv, T = 128, 1, 512
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(T, Hkv, D)
    k_new = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    v_new = torch.from_numpy(bits[::-1].copy().view(np.int16)).view(torch.bfloat16)
    NB = T // 16
    k_pool = torch.zeros((NB, Hkv, 16, D), dtype=torch.uint8)
    v_pool = torch.zeros((NB, Hkv, D, 16), dtype=torch.uint8)
    slots = torch.arange(T, dtype=torch.int64)
    ks = torch.tensor([scale], dtype=torch.float32)
    vs = torch.tensor([scale * 2.0], dtype=torch.float32)
    d = torch.device("cuda:0")
    kp, vp = k_pool.to(d), v_pool.to(d)
    ops.kv_append(k_new.to(d), v_new.to(d), slots.to(d), kp, vp, ks.to(d), vs.to(d))
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.oracle_append(k_pool.numpy(), v_pool.numpy(), storage_numpy(k_new),
                                        storage_numpy(v_new), slots.numpy(), "fp8", ks.numpy(), vs.numpy())
    assert np.array_equal(kp.cpu().numpy(), ref_k)
    assert np.array_equal(vp.cpu().numpy(), ref_v)
