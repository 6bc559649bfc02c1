"""The library's calls under HIP graph capture: they allocate nothing and
record no memory sets, so a decode step (append + decode), a shared-prefix
decode and a prefill chunk can be captured once and replayed.  Every replay,
with new queries written into the captured buffers and eager calls and
synchronisations between replays, must equal the eager result bit for bit
(same kernels, same arguments)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_cache_23_amd import ops
from paged_kv_cache_23_amd.workloads import build_workload
from tests.gpu_util import Dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    return t.numpy().view(np.uint32)


def _capture(fn):
    """Warm up on a side stream, then capture ``fn`` into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _new_q(shape, dtype, seed):
    return torch.randn(shape, generator=torch.Generator().manual_seed(seed)).to(dtype).cuda()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_decode_step_replays(kv_dtype):
    wl = build_workload("graph", [1, 40, 333, 1500, 4000, 77], 32, 8, 128, kv_dtype, seed=12, with_append=True)
    dev = Dev(wl)
    mctx = int(wl.context_lens_after.max())
    out = torch.empty_like(dev.q)
    ws = ops.new_workspace(ops.decode_workspace_bytes(dev.k_pool, dev.v_pool, 32, wl.batch, mctx,
                                                      k_scale=dev.k_scale, v_scale=dev.v_scale), dev.q.device)

    def step(q, o):
        ops.kv_append(dev.k_new, dev.v_new, dev.slots, dev.k_pool, dev.v_pool, dev.k_scale, dev.v_scale)
        ops.paged_decode(q, dev.k_pool, dev.v_pool, dev.tables_after, dev.lens_after, wl.scale, out=o,
                         k_scale=dev.k_scale, v_scale=dev.v_scale, max_context_len=mctx, workspace=ws)

    g = _capture(lambda: step(dev.q, out))
    for r in range(REPLAYS):
        q_r = _new_q(dev.q.shape, dev.q.dtype, 100 + r)
        dev.q.copy_(q_r)
        g.replay()
        torch.cuda.synchronize()
        got = _bits(out)
        eager = torch.empty_like(out)
        step(q_r, eager)   # appending the same tokens again leaves the pools unchanged
        torch.cuda.synchronize()
        assert np.array_equal(got, _bits(eager)), f"replay {r}"


def test_shared_prefix_decode_replays():
    P = 512
    rng = np.random.default_rng(13)
    wl = build_workload("graph-shared", [P + int(t) for t in rng.integers(0, 300, size=40)], 32, 8, 128, "bf16",
                        seed=13, shared_prefix=P, rng=rng)
    dev = Dev(wl)
    mctx = int(wl.context_lens.max())
    out = torch.empty_like(dev.q)
    ws = ops.new_workspace(ops.shared_decode_workspace_bytes(dev.k_pool, dev.v_pool, 32, wl.batch, mctx, P),
                           dev.q.device)

    def call(q, o):
        ops.paged_decode_shared(q, dev.k_pool, dev.v_pool, dev.tables, dev.lens, wl.scale, P, out=o,
                                max_context_len=mctx, workspace=ws)

    g = _capture(lambda: call(dev.q, out))
    for r in range(REPLAYS):
        q_r = _new_q(dev.q.shape, dev.q.dtype, 200 + r)
        dev.q.copy_(q_r)
        g.replay()
        torch.cuda.synchronize()
        got = _bits(out)
        eager = torch.empty_like(out)
        call(q_r, eager)
        torch.cuda.synchronize()
        assert np.array_equal(got, _bits(eager)), f"replay {r}"


def test_prefill_chunk_replays():
    L = 96
    wl = build_workload("graph-prefill", [L, 300, 1000], 32, 8, 128, "bf16", seed=14)
    dev = Dev(wl)
    q = _new_q((wl.batch, L, 32, 128), torch.bfloat16, 14)
    out = torch.empty_like(q)
    ws = ops.new_workspace(256, q.device)

    def call(qq, o):
        ops.paged_attention(qq, dev.k_pool, dev.v_pool, dev.tables, dev.lens, wl.scale, out=o,
                            max_context_len=1000, workspace=ws)

    g = _capture(lambda: call(q, out))
    for r in range(REPLAYS):
        q_r = _new_q(q.shape, q.dtype, 300 + r)
        q.copy_(q_r)
        g.replay()
        torch.cuda.synchronize()
        got = _bits(out)
        eager = torch.empty_like(out)
        call(q_r, eager)
        torch.cuda.synchronize()
        assert np.array_equal(got, _bits(eager)), f"replay {r}"
