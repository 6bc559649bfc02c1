#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

A step is one decode pass of one layer over the whole batch: one
pkv_paged_decode call (two kernels, split then merge; for workloads that
append, the kv_append of one token per sequence first).  Inputs are seeded synthetic data already
resident in HBM; successive steps rotate over ``--layers`` distinct copies of
the pool so that the bytes touched between reuses of one copy exceed the
256 MB Infinity Cache.

Prints ONE JSON line on stdout: KV GB/s read (the algorithmic bytes
sum_b n_b * 2 * Hkv * D * bytes/element), its share of the 8 TB/s HBM peak,
decode tokens/s (sequences / step time), the dominant kernel's roofline, and
the CPU oracle timed on this host over the same workload.

Extra modes:
  --profile-one   warm up, then launch the decode a few times (for rocprofv3)
  --copy-probe    run a plain device-to-device copy of known size (calibrates
                  the FETCH_SIZE / WRITE_SIZE counters)
  --tile-probe    the read-stream ceiling: whole tiles read at random positions
                  of a 4 GiB buffer with no arithmetic (libpkv_probe.so)
  --cow           time the copy-on-write block copy and a parallel-sampling step
  --prefill       time chunked prefill: a 10,000-token prompt in chunks of at
                  most 2048 tokens on one Llama-3-70B-shaped layer (TFLOP/s
                  against the bf16 MFMA peak)
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode KV GB/s read (% of HBM peak) + decode tokens/s, 8B-shape b64"
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["paged_kv_cache_23_amd/csrc/decode.hip", "paged_kv_cache_23_amd/csrc/split_body.h",
                  "paged_kv_cache_23_amd/csrc/tile_math.h", "paged_kv_cache_23_amd/csrc/pkv_internal.h"]
# the shared-prefix call: bf16 caches run the one-launch kernel, other dtypes
# the prefill kernel's prefix pass; both end with the decode's merge kernel
SHARED_SOURCES = {"bf16": KERNEL_SOURCES + ["paged_kv_cache_23_amd/csrc/shared.hip"],
                  "other": KERNEL_SOURCES + ["paged_kv_cache_23_amd/csrc/prefill.hip"]}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


COPY_SOURCES = ["paged_kv_cache_23_amd/csrc/copy.hip", "paged_kv_cache_23_amd/csrc/pkv_internal.h"]
APPEND_SOURCES = ["paged_kv_cache_23_amd/csrc/append.hip", "paged_kv_cache_23_amd/csrc/pkv_internal.h",
                  "paged_kv_cache_23_amd/csrc/e4m3.h"]
PREFILL_SOURCES = ["paged_kv_cache_23_amd/csrc/prefill.hip", "paged_kv_cache_23_amd/csrc/tile_math.h",
                   "paged_kv_cache_23_amd/csrc/pkv_internal.h"]


def kernel_source_hash(sources=None) -> str:
    """sha256[:16] of the kernel sources' code: '//' comments, trailing
    blanks and empty lines are dropped first, so a change to the prose alone
    keeps the recorded measurements valid."""
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = re.sub(r"//.*$", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def committed_traffic(workload: str, kind: str = "paged_decode", sources=None):
    """HBM bytes per launch unit (one pkv_paged_decode call, or one prefill
    step) from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, f"{kind}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"^source_hash:\s*(\w+)", text, re.M)
    m_bytes = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(sources):
        return None
    return float(m_bytes.group(1))


class Runner:
    """Pre-marshalled C-ABI calls for one workload on the current stream."""

    def __init__(self, wl, layers: int, workers: int = 0, identity_tables: bool = False, q_len: int = 1,
                 reread: bool = False, shared_prefix: int = 0):
        import torch
        from paged_kv_cache_23_amd import ops

        self.torch, self.ops, self.wl = torch, ops, wl
        dev = torch.device("cuda:0")
        self.q_len = int(q_len)
        if self.q_len == 1:
            self.q = wl.q.to(dev)
        else:   # L query tokens per sequence: the last L tokens of each sequence (speculative verification)
            gen = torch.Generator().manual_seed(1234)
            self.q = torch.randn((wl.batch, self.q_len, wl.num_q_heads, wl.head_dim), generator=gen).to(
                wl.q.dtype).to(dev)
        k0, v0 = wl.k_pool.to(dev), wl.v_pool.to(dev)
        # distinct copies of the pool: one per "layer" of the rotation
        self.k_pools = [k0] + [k0.clone() for _ in range(layers - 1)]
        self.v_pools = [v0] + [v0.clone() for _ in range(layers - 1)]
        self.k_scale = None if wl.k_scale is None else wl.k_scale.to(dev)
        self.v_scale = None if wl.v_scale is None else wl.v_scale.to(dev)
        self.append = wl.k_new is not None
        if self.append:
            self.k_new, self.v_new = wl.k_new.to(dev), wl.v_new.to(dev)
            self.slots = wl.slot_mapping.to(dev)
            tables, lens = wl.block_tables_after, wl.context_lens_after
        else:
            tables, lens = wl.block_tables, wl.context_lens
        self.tables, self.lens = tables.to(dev), lens.to(dev)
        if identity_tables:
            # the slab layout expressed as a table: every sequence's blocks made
            # consecutive (same bytes, same kernel, no scattered placement)
            order = [int(x) for row in tables for x in row if x >= 0]
            src = torch.tensor(order, dtype=torch.int64, device=dev)
            remap, nxt = [], 0
            for row in tables:
                k = int((row >= 0).sum())
                remap.append(list(range(nxt, nxt + k)) + [-1] * (row.numel() - k))
                nxt += k
            self.tables = torch.tensor(remap, dtype=torch.int32, device=dev)
            k0 = k0.index_select(0, src).contiguous()
            v0 = v0.index_select(0, src).contiguous()
            self.k_pools = [k0] + [k0.clone() for _ in range(layers - 1)]
            self.v_pools = [v0] + [v0.clone() for _ in range(layers - 1)]
        self.B = wl.batch
        self.max_ctx = int(lens.max())
        self.out = torch.empty_like(self.q)
        self.desc = ops.cache_desc(k0, v0, wl.num_q_heads, self.k_scale, self.v_scale, reread)
        lib = ops.library()
        self.lib = lib
        self.explicit_workers = bool(workers)
        # the shared-prefix call sizes its workers for the tails after the prefix
        self.workers = workers or lib.pkv_decode_workers(ctypes.byref(self.desc), self.B,
                                                         max(self.max_ctx - int(shared_prefix), 0))
        if self.workers <= 0:
            raise RuntimeError(f"pkv_decode_workers failed: {self.workers}")
        self.prefix = int(shared_prefix)
        if self.prefix:
            if self.q_len != 1:
                raise ValueError("the shared-prefix decode takes one query token per sequence")
            nbytes = lib.pkv_shared_decode_workspace_bytes(ctypes.byref(self.desc), self.B, self.max_ctx, self.prefix,
                                                           self.workers if self.explicit_workers else 0)
        else:
            nbytes = lib.pkv_attention_workspace_bytes(ctypes.byref(self.desc), self.B, self.q_len, self.max_ctx,
                                                       self.workers)
        if nbytes == 0:
            raise RuntimeError("pkv_attention_workspace_bytes rejected the shape")
        self.ws = ops.new_workspace(nbytes, dev)
        self.ws_bytes = self.ws.numel()
        self.kv_bytes = wl.kv_bytes(after_append=self.append)
        self.append_bytes = 0
        if self.append:   # bf16 K/V read + one code per element written
            T, Hkv, D = wl.k_new.shape
            elt = 1 if wl.kv_dtype == "fp8" else wl.k_pool.element_size()
            self.append_bytes = 2 * T * Hkv * D * (wl.k_new.element_size() + elt)

    def stream(self):
        return ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    def append_step(self, layer: int, stream):
        st = self.lib.pkv_kv_append(ctypes.byref(self.desc), self.k_new.data_ptr(), self.v_new.data_ptr(),
                                    self.slots.data_ptr(), self.slots.shape[0], self.k_pools[layer].data_ptr(),
                                    self.v_pools[layer].data_ptr(), stream)
        if st:
            raise RuntimeError(f"pkv_kv_append failed: {st}")

    def decode(self, layer: int, stream):
        workers = self.workers if self.explicit_workers else 0
        if self.prefix:
            st = self.lib.pkv_paged_decode_shared(
                ctypes.byref(self.desc), self.q.data_ptr(), self.k_pools[layer].data_ptr(),
                self.v_pools[layer].data_ptr(), self.tables.data_ptr(), self.tables.shape[1], self.lens.data_ptr(),
                self.B, self.max_ctx, self.prefix, self.wl.scale, workers, self.out.data_ptr(), self.ws.data_ptr(),
                self.ws_bytes, stream)
        elif self.q_len == 1:
            st = self.lib.pkv_paged_decode_ex(
                ctypes.byref(self.desc), self.q.data_ptr(), self.k_pools[layer].data_ptr(),
                self.v_pools[layer].data_ptr(), self.tables.data_ptr(), self.tables.shape[1], self.lens.data_ptr(),
                self.B, self.max_ctx, self.wl.scale, workers, self.out.data_ptr(), self.ws.data_ptr(),
                self.ws_bytes, stream)
        else:
            st = self.lib.pkv_paged_attention(
                ctypes.byref(self.desc), self.q.data_ptr(), self.k_pools[layer].data_ptr(),
                self.v_pools[layer].data_ptr(), self.tables.data_ptr(), self.tables.shape[1], self.lens.data_ptr(),
                self.B, self.q_len, self.max_ctx, self.wl.scale, workers, self.out.data_ptr(),
                self.ws.data_ptr(), self.ws_bytes, stream)
        if st:
            raise RuntimeError(f"paged attention call failed: {st}")

    def step(self, layer: int, stream):
        if self.append:
            self.append_step(layer, stream)
        self.decode(layer, stream)


def common_prefix_tokens(tables, lens, block_size: int) -> int:
    """Tokens in the leading blocks that every table row shares (whole blocks
    that every sequence fills)."""
    import numpy as np

    tables, lens = np.asarray(tables), np.asarray(lens)
    if tables.shape[0] == 0:
        return 0
    full = int(lens.min()) // block_size
    k = 0
    while k < full and np.all(tables[:, k] == tables[0, k]):
        k += 1
    return k * block_size


def unique_kv_bytes(wl, after_append: bool) -> int:
    """KV bytes of the distinct physical token slots a decode reads: a block
    that several sequences share counts once (with the most tokens any of them
    uses in it)."""
    import numpy as np

    tables = (wl.block_tables_after if after_append else wl.block_tables).numpy()
    lens = (wl.context_lens_after if after_append else wl.context_lens).numpy()
    bs = wl.k_pool.shape[2]
    used = {}
    for row, n in zip(tables, lens):
        nb = -(-int(n) // bs)
        for j in range(nb):
            t = min(bs, int(n) - bs * j)
            blk = int(row[j])
            if used.get(blk, 0) < t:
                used[blk] = t
    per_token = wl.kv_bytes(after_append) // max(int(np.sum(lens)), 1)
    return int(sum(used.values())) * per_token


def check_against_oracle(runner, got, sample_seqs: int = 4) -> float:
    """Max |error| of layer 0's first output ``got`` (a host copy) over a few
    sequences, against the oracle on the host copy of the pool.  Part of the
    oracle leg: run only with the CPU baseline."""
    import numpy as np

    import oracle
    from paged_kv_cache_23_amd.workloads import storage_numpy

    wl = runner.wl
    if runner.q_len > 1:
        k_pool, v_pool = storage_numpy(runner.k_pools[0].cpu()), storage_numpy(runner.v_pools[0].cpu())
        lens = wl.context_lens_after if runner.append else wl.context_lens
        nb = min(sample_seqs, wl.batch)
        ref = oracle.oracle_attention_multi(
            storage_numpy(runner.q[:nb].cpu()), wl.q_dtype, k_pool, v_pool, wl.kv_dtype,
            runner.tables[:nb].cpu().numpy(), lens[:nb].numpy(), wl.scale,
            None if wl.k_scale is None else wl.k_scale.numpy(), None if wl.v_scale is None else wl.v_scale.numpy())
        return float(np.max(np.abs(got[:nb] - ref)))
    tables = runner.tables.cpu()
    lens = wl.context_lens_after if runner.append else wl.context_lens
    k_pool, v_pool = storage_numpy(runner.k_pools[0].cpu()), storage_numpy(runner.v_pools[0].cpu())
    pairs = [(b, g) for b in range(min(sample_seqs, wl.batch)) for g in range(wl.num_kv_heads)]
    ref = oracle.oracle_decode_pairs(storage_numpy(wl.q), wl.q_dtype, k_pool, v_pool, wl.kv_dtype,
                                     tables.numpy(), lens.numpy(), wl.scale, pairs,
                                     None if wl.k_scale is None else wl.k_scale.numpy(),
                                     None if wl.v_scale is None else wl.v_scale.numpy())
    G = wl.num_q_heads // wl.num_kv_heads
    rows = np.stack([got[b, g * G:(g + 1) * G] for b, g in pairs])
    return float(np.max(np.abs(rows - ref)))


def host_cores() -> int:
    """Host cores the oracle leg runs on: this process's CPU affinity, at most
    16 (one GPU's share of the machine's cores)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


_POOL_INPUTS = None


def _oracle_pool_init(folder: str, meta: dict) -> None:
    """Oracle worker start: one BLAS thread, the inputs memory-mapped read-only."""
    global _POOL_INPUTS
    import numpy as np
    from threadpoolctl import threadpool_limits

    threadpool_limits(1)
    arrays = {name: np.load(os.path.join(folder, name + ".npy"), mmap_mode="r") for name in meta["arrays"]}
    _POOL_INPUTS = (arrays, meta)


def _oracle_ready(_) -> int:
    return os.getpid()


def _oracle_pairs_task(pairs):
    """oracle_decode_pairs, as it stands, over some (sequence, kv head) pairs."""
    import oracle

    a, m = _POOL_INPUTS
    return oracle.oracle_decode_pairs(a["q"], m["q_dtype"], a["k_pool"], a["v_pool"], m["kv_dtype"], a["tables"],
                                      a["lens"], m["scale"], pairs, a.get("k_scale"), a.get("v_scale"))


def _oracle_rows_task(rows):
    """oracle_attention_multi, as it stands, over query rows [lo, hi) of one
    chunk (they see the first n - L + hi tokens)."""
    import oracle

    a, m = _POOL_INPUTS
    lo, hi = rows
    return oracle.oracle_attention_multi(a["q"][:, lo:hi], m["q_dtype"], a["k_pool"], a["v_pool"], m["kv_dtype"],
                                         a["tables"], [m["n"] - m["L"] + hi], m["scale"], a.get("k_scale"),
                                         a.get("v_scale"))


class OraclePool:
    """The oracle on the host's cores: spawned worker processes (they never
    touch the GPU), each with one BLAS thread, sharing the inputs through
    memory-mapped files; tasks are handed out one at a time, longest first."""

    def __init__(self, arrays: dict, meta: dict, workers: int):
        import multiprocessing
        import tempfile

        import numpy as np

        self._dir = tempfile.TemporaryDirectory(prefix="pkv_oracle_")
        names = []
        for name, arr in arrays.items():
            if arr is not None:
                np.save(os.path.join(self._dir.name, name + ".npy"), np.ascontiguousarray(arr))
                names.append(name)
        self.workers = workers
        ctx = multiprocessing.get_context("spawn")
        self._pool = ctx.Pool(workers, initializer=_oracle_pool_init,
                              initargs=(self._dir.name, dict(meta, arrays=names)))
        self._pool.map(_oracle_ready, range(workers), chunksize=1)

    def map(self, fn, tasks):
        return self._pool.map(fn, tasks, chunksize=1)

    def close(self) -> None:
        self._pool.close()
        self._pool.join()
        self._dir.cleanup()


def cpu_baseline(wl, min_seconds: float = 10.0, max_reps: int = 400):
    """The oracle, as it stands, on this host's cores: whole decode steps of
    the workload (every sequence and kv head; the (sequence, kv head) pairs
    shared out over a process pool), repeated until min_seconds."""
    from paged_kv_cache_23_amd.workloads import storage_numpy

    lens = wl.context_lens.numpy()
    pool = OraclePool(dict(q=storage_numpy(wl.q), k_pool=storage_numpy(wl.k_pool), v_pool=storage_numpy(wl.v_pool),
                           tables=wl.block_tables.numpy(), lens=lens,
                           k_scale=None if wl.k_scale is None else wl.k_scale.numpy(),
                           v_scale=None if wl.v_scale is None else wl.v_scale.numpy()),
                      dict(q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype, scale=wl.scale), host_cores())
    try:
        pairs = sorted(((b, g) for b in range(wl.batch) for g in range(wl.num_kv_heads)), key=lambda p: -lens[p[0]])
        tasks = [[p] for p in pairs]
        pool.map(_oracle_pairs_task, tasks)          # first pass: page the inputs in
        reps, t0 = 0, time.perf_counter()
        while reps < max_reps:
            pool.map(_oracle_pairs_task, tasks)
            reps += 1
            if time.perf_counter() - t0 >= min_seconds:
                break
        sec = (time.perf_counter() - t0) / reps
    finally:
        pool.close()
    return {
        "value": round(wl.kv_bytes() / sec / 1e9, 4),
        "unit": "GB/s",
        "cores": pool.workers,
        "kind": "oracle",
        "sample": f"whole {wl.name} decode steps (all {wl.batch} sequences x {wl.num_kv_heads} kv heads, "
                  f"{wl.kv_bytes() / 1e6:.0f} MB of KV) in fp64 NumPy, the pairs shared out over "
                  f"{pool.workers} host processes of one thread each, {reps} repetitions, {sec:.3f} s each",
        "seconds_per_step": round(sec, 4),
        "decode_tokens_per_s": round(wl.batch / sec, 2),
    }


def make_runner(args):
    """The workload and its pre-marshalled calls, in the launch configuration
    that the benchmark times (and that --profile-one profiles)."""
    from paged_kv_cache_23_amd import workloads as W

    wl = W.WORKLOADS[args.workload](block_size=args.block_size)
    log(f"workload {wl.name}: B={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} D={wl.head_dim} "
        f"kv={wl.kv_dtype} blocks={wl.num_blocks} KV={wl.kv_bytes() / 1e6:.1f} MB")
    after = wl.k_new is not None
    # a scheduler knows from its reference counts whether the batch shares
    # blocks; here: when the distinct token slots are fewer than 90% of those read
    shares = unique_kv_bytes(wl, after) < 0.9 * wl.kv_bytes(after_append=after)
    prefix = 0
    if args.shared:
        prefix = common_prefix_tokens((wl.block_tables_after if after else wl.block_tables).numpy(),
                                      (wl.context_lens_after if after else wl.context_lens).numpy(), args.block_size)
        if prefix == 0:
            raise SystemExit(f"--shared: the tables of {wl.name} share no leading block")
        log(f"shared-prefix decode: {prefix} tokens ({prefix // args.block_size} blocks) read once per call")
    # the shared-prefix call reads the prefix once and every tail once: streamed loads
    reread = (shares and not prefix) if args.reread == "auto" else args.reread == "on"
    runner = Runner(wl, args.layers, args.workers, args.identity_tables, args.q_len, reread, prefix)
    return wl, runner, prefix, reread


def run_bench(args) -> dict:
    import numpy as np
    import torch

    wl, runner, prefix, reread = make_runner(args)
    streamed = not reread and args.block_size <= 32
    loads = "streamed (non-temporal)" if streamed else (
        "cached (PKV_KV_REREAD: blocks shared)" if reread else "cached (blocks above 32 tokens)")
    log(f"workers={runner.workers} waves, workspace={runner.ws_bytes} B, layers={args.layers}, K/V loads {loads}")
    torch.cuda.synchronize()

    # one step on layer 0 whose output is kept for the oracle leg's check
    s = runner.stream()
    runner.step(0, s)
    torch.cuda.synchronize()
    out0 = runner.out.float().cpu().numpy().astype(np.float64)

    L = args.layers
    for i in range(args.warmup):
        runner.step(i % L, s)
    torch.cuda.synchronize()

    # timed region: K steps, events only at its two ends
    K = args.steps
    start_ev = torch.cuda.Event(enable_timing=True)
    end_ev = torch.cuda.Event(enable_timing=True)
    t_wall0 = time.perf_counter()
    start_ev.record()
    for i in range(K):
        runner.step(i % L, s)
    end_ev.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    total_ms = start_ev.elapsed_time(end_ev)
    ms_per_step = total_ms / K

    # per-call durations of the decode (split + merge kernels): the same
    # steps, HIP events around each call on the stream its kernels run on
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        layer = i % L
        if runner.append:
            runner.append_step(layer, s)
        ev[i][0].record()
        runner.decode(layer, s)
        ev[i][1].record()
    torch.cuda.synchronize()
    part_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    log(f"{K} steps: {total_ms:.3f} ms on the stream, {wall * 1e3:.3f} ms wall ({ms_per_step * 1e3:.1f} us/step); "
        f"decode call mean {part_ms.mean() * 1e3:.1f} us (p10 {np.percentile(part_ms, 10) * 1e3:.1f}, "
        f"p90 {np.percentile(part_ms, 90) * 1e3:.1f})")

    step_bytes = runner.kv_bytes + runner.append_bytes
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    unique = unique_kv_bytes(wl, runner.append)
    # the shared-prefix call's algorithmic bytes are the distinct slots: the
    # prefix once plus every tail
    algo = unique if prefix else runner.kv_bytes
    kern_gbs = algo / (part_ms.mean() * 1e-3) / 1e9
    one_launch = wl.kv_dtype == "bf16"
    traffic = (committed_traffic(wl.name, "paged_decode_shared", SHARED_SOURCES["bf16" if one_launch else "other"])
               if prefix else committed_traffic(wl.name))
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 kv / bf16 q"}[wl.kv_dtype],
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: single-layer paged decode, batch {wl.batch}, {wl.num_q_heads} q / "
                        f"{wl.num_kv_heads} kv heads, head_dim {wl.head_dim}, {args.block_size}-token blocks, "
                        f"shuffled pool, {args.layers}-layer pool rotation",
            "batch": wl.batch,
            "context_tokens": int((wl.context_lens_after if runner.append else wl.context_lens).sum()),
            "kv_bytes_per_step": step_bytes,
            "worker_waves": runner.workers,
            "kv_loads": loads,
            "shared_prefix_tokens": prefix,
        },
        "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4),
        "unique_kv_bytes_per_step": unique,
        "unique_kv_gbs": round(unique / (ms_per_step * 1e-3) / 1e9, 2),
        "decode_tokens_per_s": round(wl.batch * args.q_len / (ms_per_step * 1e-3), 1),
        "query_tokens_per_seq": args.q_len,
        "max_abs_err_sampled": None,
        "roofline": {
            "kernel": (("pkv_paged_decode_shared (decode_shared_kernel: tail walk and prefix waves in one "
                        "launch; shared_merge_kernel)" if one_launch else
                        "pkv_paged_decode_shared (prefill_kernel over the prefix + decode_split_kernel + "
                        "decode_merge_kernel)") if prefix else
                       "pkv_paged_decode (decode_split_kernel + decode_merge_kernel)"),
            "bound": "hbm",
            "achieved": round(kern_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": algo,
            "mean_call_us": round(float(part_ms.mean()) * 1e3, 2),
            "call_us_p10_p50_p90": [round(float(np.percentile(part_ms, q)) * 1e3, 2) for q in (10, 50, 90)],
        },
    }
    if not args.no_cpu_baseline:
        # the oracle leg: the sampled check of layer 0's first output, then
        # the oracle timed on the host
        err = check_against_oracle(runner, out0)
        log(f"parity on sampled sequences: max|err| = {err:.3g}")
        result["max_abs_err_sampled"] = err
        log("timing the CPU oracle on the host ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    return result


def profile_one(args) -> None:
    import torch

    wl, runner, _, _ = make_runner(args)
    s = runner.stream()
    for i in range(args.warmup):
        runner.step(i % args.layers, s)
    torch.cuda.synchronize()
    for i in range(args.steps):
        runner.step(i % args.layers, s)
    torch.cuda.synchronize()
    log(f"profiled {args.steps} steps of {wl.name} ({runner.workers} workers, {runner.kv_bytes} KV bytes/step)")


def copy_probe(args) -> None:
    import torch

    n = 1 << 30   # 1 GiB read + 1 GiB written per copy
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {n} bytes {args.steps} times")


def tile_probe(args) -> dict:
    """The read-stream ceiling: libpkv_probe.so reads whole tiles at random
    positions of a 4 GiB buffer (the decode's access pattern with no
    arithmetic; the decode reads one 4 KiB (bf16) or 2 KiB (fp8) tile per
    (block, kv head) for K and one for V), over tile sizes, KiB in flight per
    wave, ordinary and non-temporal loads and one or two waves per SIMD; also
    the same tiles read in order.  Each line: GB/s over 10 launches timed with
    HIP events on the launch stream."""
    import numpy as np
    import torch

    from paged_kv_cache_23_amd.build import PROBE_PATH

    lib = ctypes.CDLL(PROBE_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.pkv_probe_read_tiles.restype = ctypes.c_int
    lib.pkv_probe_read_tiles.argtypes = [P, SZ, P, I64, I32, I32, I32, I32, P, P]
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(4 * cus * 2 * 64, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.current_stream()
    rng = np.random.default_rng(0)
    rows = []
    for tile_kib in args.probe_tiles:
        n = nbytes // (tile_kib << 10)
        ids = {"random": torch.from_numpy(rng.permutation(n).astype(np.int32)).cuda(),
               "in order": torch.arange(n, dtype=torch.int32, device="cuda:0")}
        for order, t in ids.items():
            for waves_per_simd in (1, 2):
                for kib in (4, 8, 16, 32):
                    for nt in (1, 0):
                        if order == "in order" and (kib != 16 or waves_per_simd != 1):
                            continue
                        waves = 4 * cus * waves_per_simd

                        def launch():
                            st = lib.pkv_probe_read_tiles(buf.data_ptr(), nbytes, t.data_ptr(), n, tile_kib, kib,
                                                          waves, nt, sink.data_ptr(), ctypes.c_void_p(s.cuda_stream))
                            if st != 0:
                                raise RuntimeError(f"pkv_probe_read_tiles: status {st}")
                        for _ in range(2):
                            launch()
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(s)
                        for _ in range(10):
                            launch()
                        e1.record(s)
                        torch.cuda.synchronize()
                        us = e0.elapsed_time(e1) / 10 * 1e3
                        rows.append({"tile_kib": tile_kib, "order": order, "waves_per_simd": waves_per_simd,
                                     "kib_in_flight_per_wave": kib, "loads": "non-temporal" if nt else "cached",
                                     "us": round(us, 1), "GB/s": round(nbytes / us / 1e3, 1)})
                        log(f"tiles {tile_kib} KiB {order:8s} {waves_per_simd} wave/SIMD {kib:2d} KiB in flight "
                            f"{'nt ' if nt else 'ord'}: {nbytes / us / 1e3:8.1f} GB/s")
    best = max((r for r in rows if r["order"] == "random"), key=lambda r: r["GB/s"])
    return {"metric": "random-tile read stream (probe, no arithmetic)", "value": best["GB/s"], "unit": "GB/s",
            "n_gpus": 1, "higher_is_better": True, "data": "synthetic",
            "config": {"workload": "4 GiB buffer read once per launch as whole tiles in a random permutation",
                       "best": best}, "rows": rows}


def cow_bench(args) -> dict:
    """Copy-on-write: pkv_copy_blocks at the parallel-sampling shape (8 samples
    of a 2005-token prompt: one shared 5-token block copied per sample, 32 KiB
    per pool at bf16) and at a large batch of pairs, then one whole sampling
    step (copy + append + decode of the prompt and its 8 samples)."""
    import numpy as np
    import torch

    from paged_kv_cache_23_amd import ops
    from paged_kv_cache_23_amd.workloads import cow_sampling

    dev = torch.device("cuda:0")
    sc = cow_sampling("cow-8", prompt_tokens=2005, samples=8, new_tokens=1, num_q_heads=32,
                      num_kv_heads=8, head_dim=128, kv_dtype="bf16", seed=44)
    kp, vp = sc.k_pool.to(dev), sc.v_pool.to(dev)
    st = sc.steps[0]
    src, dst = st.copy_src.to(dev), st.copy_dst.to(dev)
    block_bytes = sc.num_kv_heads * 16 * sc.head_dim * 2

    def timed(fn, reps):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3   # us

    small_us = timed(lambda: ops.copy_blocks(kp, vp, src, dst), 500)
    small_bytes = 2 * 2 * len(st.copy_src) * block_bytes            # read + write, K and V
    # a large batch: 4096 pairs over a 16384-block pool (distinct, disjoint)
    NB = 16384
    big_k = torch.empty((NB, 8, 16, 128), dtype=torch.bfloat16, device=dev).normal_()
    big_v = torch.empty((NB, 8, 128, 16), dtype=torch.bfloat16, device=dev).normal_()
    perm = torch.from_numpy(np.random.default_rng(7).permutation(NB).astype(np.int32)).to(dev)
    bsrc, bdst = perm[:4096].contiguous(), perm[4096:8192].contiguous()
    big_us = timed(lambda: ops.copy_blocks(big_k, big_v, bsrc, bdst), 50)
    big_bytes = 2 * 2 * 4096 * block_bytes
    # one whole sampling step on the scenario (the copy is idempotent to repeat)
    q, tables, lens = sc.q.to(dev), sc.block_tables.to(dev), sc.context_lens.to(dev)
    kn, vn, slots = st.k_new.to(dev), st.v_new.to(dev), st.slot_mapping.to(dev)
    out = torch.empty_like(q)
    mctx = int(sc.context_lens.max())
    ws = ops.new_workspace(ops.decode_workspace_bytes(kp, vp, 32, q.shape[0], mctx), dev)

    def step():
        ops.copy_blocks(kp, vp, src, dst)
        ops.kv_append(kn, vn, slots, kp, vp)
        ops.paged_decode(q, kp, vp, tables, lens, sc.scale, out=out, max_context_len=mctx, workspace=ws)
    step_us = timed(step, 200)
    log(f"copy 8 pairs: {small_us:.2f} us; copy 4096 pairs: {big_us:.1f} us "
        f"({big_bytes / big_us / 1e3:.0f} GB/s); sampling step: {step_us:.1f} us")
    big_gbs = big_bytes / big_us / 1e3
    result = {
        "metric": "copy-on-write block copy GB/s (pkv_copy_blocks, read + write) and parallel-sampling step",
        "value": round(big_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": 50,
        "warmup": 10,
        "ms_per_step": round(big_us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "copy_8_pairs_us": round(small_us, 2),
        "copy_8_pairs_bytes": small_bytes,
        "copy_4096_pairs_us": round(big_us, 2),
        "copy_4096_pairs_bytes": big_bytes,
        "copy_4096_pairs_gbs": round(big_bytes / big_us / 1e3, 1),
        "copy_4096_pairs_hbm_frac": round(big_bytes / big_us / 1e3 / HBM_PEAK_GBS, 4),
        "sampling_step_us": round(step_us, 2),
        "config": {"workload": "4096 block pairs of a 16384-block bf16 pool (8 kv heads, 16 tokens, head_dim 128: "
                               "32 KiB per block and pool); the sampling step: 8 samples of a 2005-token prompt, "
                               "32 q / 8 kv heads"},
        "roofline": {
            "kernel": "copy_blocks_kernel (4096 pairs)",
            "bound": "hbm",
            "achieved": round(big_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(big_gbs / HBM_PEAK_GBS, 4),
            "traffic": committed_traffic("copy-4096", "copy_blocks_kernel", COPY_SOURCES),
            "algorithmic_bytes_per_launch": big_bytes,
            "mean_call_us": round(big_us, 2),
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the host ...")
        result["cpu_baseline"] = cow_cpu_baseline(args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    return result


def cow_cpu_baseline(min_seconds: float):
    """The oracle's block copy on this host over a bounded sample: 512 pairs
    of a 2048-block bf16 pool per call, repeated for min_seconds."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    rng = np.random.default_rng(8)
    NB, pairs = 2048, 512
    kp = rng.integers(0, 1 << 16, size=(NB, 8, 16, 128), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, size=(NB, 8, 128, 16), dtype=np.uint16)
    perm = rng.permutation(NB)
    src, dst = perm[:pairs], perm[pairs:2 * pairs]
    block_bytes = 8 * 16 * 128 * 2
    reps, t0 = 0, time.perf_counter()
    with threadpool_limits(1):
        while reps == 0 or time.perf_counter() - t0 < min_seconds:
            oracle.oracle_copy_blocks(kp, vp, src, dst)
            reps += 1
    sec = time.perf_counter() - t0
    return {
        "value": round(reps * 2 * 2 * pairs * block_bytes / sec / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{pairs} block copies (K and V, 32 KiB per block and pool) in a {NB}-block bf16 pool through "
                  f"oracle_copy_blocks (which copies the whole pool first), {reps} calls, {sec:.1f} s on one "
                  f"host thread; value counts the copied blocks' read + write bytes",
    }


def append_bench(args) -> dict:
    """kv_append on its own: 65,536 new tokens of a Llama-3-8B layer (8 kv
    heads, head_dim 128) into consecutive slots (a prefill chunk's appends,
    the line's value), plus scattered slots at 65,536, 4,096 and 256 tokens
    (decode steps append one token per sequence into its own block)."""
    import numpy as np
    import torch

    from paged_kv_cache_23_amd import ops
    from paged_kv_cache_23_amd.workloads import storage_numpy

    dev = torch.device("cuda:0")
    kv = args.kv_dtype
    Hkv, D, bs = 8, 128, args.block_size
    fp8 = kv == "fp8"
    elt = {"f32": 4, "bf16": 2, "fp8": 1}[kv]
    in_elt = 4 if kv == "f32" else 2
    pool_dtype = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[kv]
    new_dtype = torch.float32 if kv == "f32" else torch.bfloat16
    scales = (torch.full((Hkv,), 4.0 / 448.0, dtype=torch.float32, device=dev),) * 2 if fp8 else (None, None)
    gen = torch.Generator().manual_seed(9)
    rng = np.random.default_rng(9)

    def case(T, pattern, reps):
        NB = (T // bs + 8) if pattern == "consecutive" else 2 * T + 8
        kp = torch.zeros((NB, Hkv, bs, D), dtype=pool_dtype, device=dev)
        vp = torch.zeros((NB, Hkv, D, bs), dtype=pool_dtype, device=dev)
        kn = torch.randn((T, Hkv, D), generator=gen).to(new_dtype).to(dev)
        vn = torch.randn((T, Hkv, D), generator=gen).to(new_dtype).to(dev)
        if pattern == "consecutive":
            slots = np.arange(T, dtype=np.int64) + 3 * bs
        else:
            slots = rng.permutation(NB)[:T].astype(np.int64) * bs + rng.integers(0, bs, size=T)
        sl = torch.from_numpy(slots).to(dev)
        call = lambda: ops.kv_append(kn, vn, sl, kp, vp, *scales)
        for _ in range(5):
            call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            call()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / reps * 1e3
        nbytes = T * Hkv * D * 2 * (in_elt + elt)   # K and V: read the new values, write the pool
        log(f"append {kv} T={T} {pattern}: {us:.1f} us per call, {nbytes / us / 1e3:.1f} GB/s")
        return us, nbytes, (kp, vp, kn, vn, slots)

    us, nbytes, keep = case(65536, "consecutive", args.steps)
    others = {f"{p}_{T}": case(T, p, args.steps)[:2] for T, p in ((65536, "scattered"), (4096, "scattered"),
                                                                     (256, "scattered"))}
    gbs = nbytes / us / 1e3
    result = {
        "metric": "kv_append GB/s (new K/V read + pool written), 65,536 tokens into consecutive slots",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": 5,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 kv / bf16 input"}[kv],
        "data": "synthetic",
        "config": {"workload": f"65,536 new tokens, 8 kv heads, head_dim 128, {bs}-token blocks, {kv} cache"},
        "scattered_us": {k: round(v[0], 2) for k, v in others.items()},
        "scattered_gbs": {k: round(v[1] / v[0] / 1e3, 1) for k, v in others.items()},
        "max_abs_err_sampled": None,
        "roofline": {
            "kernel": f"append_kernel<{kv}, 128>",
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": (committed_traffic(f"append-65536-{kv}", "append_kernel", APPEND_SOURCES)
                        if bs == 16 else None),
            "algorithmic_bytes_per_launch": nbytes,
            "mean_call_us": round(us, 2),
        },
    }
    if not args.no_cpu_baseline:
        # the oracle leg: the first 512 tokens' slots compared bit for bit,
        # then the oracle's append timed on the host
        import oracle
        from threadpoolctl import threadpool_limits

        kp, vp, kn, vn, slots = keep
        n = 512
        sub = slice(0, (n + 3 * bs) // bs)   # the blocks that only these tokens fill
        k0 = np.zeros(storage_numpy(kp[sub].cpu()).shape, dtype=storage_numpy(kp[sub].cpu()).dtype)
        v0 = np.zeros(storage_numpy(vp[sub].cpu()).shape, dtype=k0.dtype)
        sc = (None, None) if not fp8 else tuple(x.cpu().numpy() for x in scales)
        ref_k, ref_v = oracle.oracle_append(k0, v0, storage_numpy(kn[:n].cpu()), storage_numpy(vn[:n].cpu()),
                                            slots[:n], kv, *sc)
        exact = bool(np.array_equal(storage_numpy(kp[sub].cpu()), ref_k) and
                     np.array_equal(storage_numpy(vp[sub].cpu()), ref_v))
        log(f"first {n} tokens' slots equal the oracle's append: {exact}")
        result["max_abs_err_sampled"] = 0.0 if exact else None
        result["append_bit_exact_sampled"] = exact
        reps, t0 = 0, time.perf_counter()
        with threadpool_limits(1):
            while reps == 0 or time.perf_counter() - t0 < args.cpu_seconds:
                oracle.oracle_append(k0, v0, storage_numpy(kn[:n].cpu()), storage_numpy(vn[:n].cpu()), slots[:n], kv,
                                     *sc)
                reps += 1
        sec = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(reps * n * Hkv * D * 2 * (in_elt + elt) / sec / 1e9, 4),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"oracle_append of {n} tokens into a {k0.shape[0]}-block pool (which it copies first), "
                      f"{reps} calls, {sec:.1f} s on one host thread",
        }
    else:
        result["cpu_baseline"] = None
    return result


MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3


class PrefillRunner:
    """The chunk steps of one prompt's chunked prefill, pre-marshalled."""

    def __init__(self, block_size: int = 16, kv_dtype: str = "bf16"):
        import torch
        from paged_kv_cache_23_amd import ops
        from paged_kv_cache_23_amd.workloads import prefill_chunks

        self.torch, self.ops = torch, ops
        dev = torch.device("cuda:0")
        self.kv_dtype = kv_dtype
        self.steps = prefill_chunks(block_size=block_size, kv_dtype=kv_dtype)
        wl = self.steps[0].wl
        self.wl = wl
        self.k_pool, self.v_pool = wl.k_pool.to(dev), wl.v_pool.to(dev)
        self.tables = wl.block_tables.to(dev)
        self.q = [s.q.to(dev) for s in self.steps]
        self.out = [torch.empty_like(q) for q in self.q]
        self.lens = [s.wl.context_lens.to(dev) for s in self.steps]
        self.n = [int(s.wl.context_lens[0]) for s in self.steps]
        self.flops = [s.flops() for s in self.steps]
        self.k_scale = None if wl.k_scale is None else wl.k_scale.to(dev)
        self.v_scale = None if wl.v_scale is None else wl.v_scale.to(dev)
        self.desc = ops.cache_desc(self.k_pool, self.v_pool, wl.num_q_heads, self.k_scale, self.v_scale)
        self.lib = ops.library()
        self.ws = ops.new_workspace(256, dev)

    def chunk(self, k: int, stream):
        q = self.q[k]
        st = self.lib.pkv_paged_attention(
            ctypes.byref(self.desc), q.data_ptr(), self.k_pool.data_ptr(), self.v_pool.data_ptr(),
            self.tables.data_ptr(), self.tables.shape[1], self.lens[k].data_ptr(), 1, q.shape[1], self.n[k],
            self.wl.scale, 0, self.out[k].data_ptr(), self.ws.data_ptr(), 256, stream)
        if st:
            raise RuntimeError(f"pkv_paged_attention failed: {st}")

    def step(self, stream):
        for k in range(len(self.steps)):
            self.chunk(k, stream)


def prefill_parity(runner, outs, rows: int = 4) -> float:
    """Max |error| of a few sampled query rows of every chunk's first output
    (``outs``, host copies) against the oracle.  Part of the oracle leg."""
    import numpy as np

    import oracle
    from paged_kv_cache_23_amd.workloads import storage_numpy

    wl = runner.wl
    kp, vp = storage_numpy(wl.k_pool), storage_numpy(wl.v_pool)
    worst = 0.0
    for k, s in enumerate(runner.steps):
        L = s.q.shape[1]
        got = outs[k]
        for i in np.linspace(0, L - 1, rows).astype(int):
            lens = np.array([runner.n[k] - L + 1 + int(i)], dtype=np.int32)
            ref = oracle.oracle_decode(storage_numpy(s.q[:, i]), wl.q_dtype, kp, vp, wl.kv_dtype,
                                       wl.block_tables.numpy(), lens, wl.scale, *_scales(wl))
            worst = max(worst, float(np.max(np.abs(got[:, i] - ref))))
    return worst


def _scales(wl):
    """The fp8 pools' per-head scales as host arrays (None, None otherwise)."""
    return (None if wl.k_scale is None else wl.k_scale.numpy(), None if wl.v_scale is None else wl.v_scale.numpy())


def prefill_cpu_baseline(runner, min_seconds: float):
    """The oracle on this host's cores over a bounded sample: the query rows of
    the last chunk (each sees about 8,200 tokens), four rows per task over a
    process pool, rows added until min_seconds; reported as TFLOP/s of the
    same causal flop count."""
    from paged_kv_cache_23_amd.workloads import storage_numpy

    wl, s = runner.wl, runner.steps[-1]
    L, n = s.q.shape[1], runner.n[-1]
    ks, vs = _scales(wl)
    pool = OraclePool(dict(q=storage_numpy(s.q), k_pool=storage_numpy(wl.k_pool), v_pool=storage_numpy(wl.v_pool),
                           tables=wl.block_tables.numpy(), k_scale=ks, v_scale=vs),
                      dict(q_dtype=wl.q_dtype, kv_dtype=wl.kv_dtype, scale=wl.scale, n=n, L=L), host_cores())
    try:
        rows = 4
        pool.map(_oracle_rows_task, [(i * rows, (i + 1) * rows) for i in range(pool.workers)])   # page in
        done, flops, t0 = 0, 0, time.perf_counter()
        while done < L and time.perf_counter() - t0 < min_seconds:
            batch = [(lo, min(L, lo + rows)) for lo in range(done, min(L, done + rows * pool.workers), rows)]
            pool.map(_oracle_rows_task, batch)
            hi = batch[-1][1]
            flops += sum(4 * wl.num_q_heads * wl.head_dim * (n - L + 1 + i) for i in range(done, hi))
            done = hi
        sec = time.perf_counter() - t0
    finally:
        pool.close()
    return {
        "value": round(flops / sec / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": pool.workers,
        "kind": "oracle",
        "sample": f"first {done} query rows of the last chunk (n = {n}, {wl.num_q_heads} q heads) through "
                  f"oracle_attention_multi in fp64 NumPy, {rows} rows per task over {pool.workers} host "
                  f"processes of one thread each, {sec:.1f} s",
    }


def prefill_bench(args) -> dict:
    """Chunked prefill: the 10,000-token prompt of the pages' worked example,
    five chunk calls per step, each over every chunk before it."""
    import numpy as np
    import torch

    runner = PrefillRunner(args.block_size, args.kv_dtype)
    wl = runner.wl
    flops = sum(runner.flops)
    kv = args.kv_dtype
    # fp8 codes are widened to bf16 for the bf16 MFMA; a float32 cache runs
    # the float32 MFMA (dense peak 157.3 TFLOP/s)
    peak = MFMA_F32_PEAK_TFLOPS if kv == "f32" else MFMA_BF16_PEAK_TFLOPS
    mfma = "f32" if kv == "f32" else "bf16"
    log(f"prefill {wl.name}: chunks {[int(q.shape[1]) for q in runner.q]} over n = {runner.n}, "
        f"Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} D={wl.head_dim}, {flops / 1e9:.1f} GFLOP per step")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    runner.step(s)
    torch.cuda.synchronize()
    outs0 = [o.float().cpu().numpy().astype(np.float64) for o in runner.out]   # for the oracle leg's check
    for _ in range(args.warmup):
        runner.step(s)
    torch.cuda.synchronize()
    K = args.steps
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(K):
        runner.step(s)
    b.record()
    torch.cuda.synchronize()
    ms_per_step = a.elapsed_time(b) / K
    # per-call durations, HIP events around each chunk call on its stream
    nck = len(runner.steps)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K * nck)]
    for i in range(K):
        for k in range(nck):
            ev[i * nck + k][0].record()
            runner.chunk(k, s)
            ev[i * nck + k][1].record()
    torch.cuda.synchronize()
    call_ms = np.array([e[0].elapsed_time(e[1]) for e in ev]).reshape(K, nck)
    mean_call = call_ms.mean(axis=0)
    per_chunk = [round(float(f / (m * 1e-3) / 1e12), 1) for f, m in zip(runner.flops, mean_call)]
    kern_tflops = flops / (mean_call.sum() * 1e-3) / 1e12
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    log(f"{K} steps: {ms_per_step * 1e3:.1f} us/step, {tflops:.1f} TFLOP/s; per chunk call (us) "
        f"{[round(float(m) * 1e3, 1) for m in mean_call]}, TFLOP/s {per_chunk}")
    result = {
        "metric": f"chunked-prefill paged attention TFLOP/s ({mfma} MFMA)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 kv / bf16 q"}[kv],
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: one layer (64 q / 8 kv heads, head_dim 128, {kv} cache, {args.block_size}-token "
                        f"blocks, shuffled pool) prefilling a 10,000-token prompt in chunks of "
                        f"{[int(q.shape[1]) for q in runner.q]}, each attending causally to all chunks before it",
            "flops_per_step": flops,
            "prefill_tokens_per_step": int(sum(q.shape[1] for q in runner.q)),
        },
        "prefill_tokens_per_s": round(sum(q.shape[1] for q in runner.q) / (ms_per_step * 1e-3), 1),
        "max_abs_err_sampled": None,
        "per_chunk_call_us": [round(float(m) * 1e3, 2) for m in mean_call],
        "per_chunk_tflops": per_chunk,
        "roofline": {
            "kernel": f"prefill_kernel<{kv}, 128>",
            "bound": "mfma",
            "achieved": round(kern_tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(kern_tflops / peak, 4),
            # the committed counters were taken on the bf16 cache
            "traffic": committed_traffic(wl.name, "prefill_kernel", PREFILL_SOURCES) if kv == "bf16" else None,
            "traffic_unit": "HBM bytes per step (five calls)",
            "algorithmic_flops_per_step": flops,
            "mean_step_kernel_us": round(float(mean_call.sum()) * 1e3, 2),
        },
    }
    if not args.no_cpu_baseline:
        err = prefill_parity(runner, outs0)
        log(f"parity on sampled rows: max|err| = {err:.3g}")
        result["max_abs_err_sampled"] = err
        log("timing the CPU oracle on the host ...")
        result["cpu_baseline"] = prefill_cpu_baseline(runner, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    return result


def prefill_profile(args) -> None:
    import torch

    runner = PrefillRunner(args.block_size, args.kv_dtype)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(args.warmup + args.steps):
        runner.step(s)
    torch.cuda.synchronize()
    log(f"profiled {args.warmup + args.steps} prefill steps")


def main() -> int:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="llama3-8b-b64")
    p.add_argument("--layers", type=int, default=4)
    p.add_argument("--workers", type=int, default=0, help="decode worker waves (0: the library's choice)")
    p.add_argument("--identity-tables", action="store_true",
                   help="store each sequence's blocks consecutively (the slab layout as a table)")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--profile-one", action="store_true")
    p.add_argument("--copy-probe", action="store_true")
    p.add_argument("--tile-probe", action="store_true",
                   help="measure the random-tile read ceiling with the probe library instead")
    p.add_argument("--probe-tiles", type=int, nargs="+", default=[1, 2, 4, 8],
                   help="tile sizes (KiB) for --tile-probe")
    p.add_argument("--cow", action="store_true", help="time the copy-on-write block copy instead")
    p.add_argument("--block-size", type=int, default=16, help="tokens per cache block (16, 32, 64, 128, 256)")
    p.add_argument("--reread", choices=["auto", "on", "off"], default="auto",
                   help="PKV_KV_REREAD hint: auto = on when the tables share blocks")
    p.add_argument("--shared", action="store_true",
                   help="decode through pkv_paged_decode_shared: the tables' common leading blocks read once")
    p.add_argument("--kv-dtype", choices=["bf16", "fp8", "f32"], default="bf16",
                   help="cache dtype of the --prefill and --append workloads")
    p.add_argument("--append", action="store_true", help="time kv_append on its own instead")
    p.add_argument("--prefill", action="store_true",
                   help="time chunked prefill (a 10,000-token prompt in 2048-token chunks) instead")
    p.add_argument("--q-len", type=int, default=1,
                   help="query tokens per sequence (speculative verification); 1 is the decode")
    args = p.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr, flush=True)
        return 2
    if args.copy_probe:
        copy_probe(args)
        return 0
    if args.tile_probe:
        print(json.dumps(tile_probe(args)), flush=True)
        return 0
    if args.prefill and args.profile_one:
        prefill_profile(args)
        return 0
    if args.profile_one:
        profile_one(args)
        return 0
    if args.prefill:
        print(json.dumps(prefill_bench(args)), flush=True)
        return 0
    if args.cow:
        print(json.dumps(cow_bench(args)), flush=True)
        return 0
    if args.append:
        print(json.dumps(append_bench(args)), flush=True)
        return 0
    result = run_bench(args)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
