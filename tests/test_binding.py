"""Host-side logic of the ctypes binding (no GPU needed)."""

from __future__ import annotations

import contextlib

import torch

from paged_kv_cache_23_amd import ops


def test_temporary_workspace_is_allocated_on_the_kernels_stream(monkeypatch):
    """A per-call workspace is allocated under the stream the call's kernels
    run on (so torch's caching allocator cannot give it to another stream
    while they may still be using it); with no stream, on the current one."""
    entered = []

    class FakeExternal:
        def __init__(self, handle, device=None):
            self.handle = handle

    @contextlib.contextmanager
    def fake_stream_ctx(s):
        entered.append(s)
        yield

    monkeypatch.setattr(torch.cuda, "ExternalStream", FakeExternal)
    monkeypatch.setattr(torch.cuda, "stream", fake_stream_ctx)
    ws = ops._temp_workspace(100, "cpu", 1234)
    assert ws.numel() >= 100 and len(entered) == 1 and entered[0].handle == 1234

    class HasHandle:
        cuda_stream = 77
    ops._temp_workspace(16, "cpu", HasHandle())
    assert entered[-1].handle == 77
    ops._temp_workspace(16, "cpu", None)
    assert len(entered) == 2
