"""Seeded synthetic workloads shaped like the pages' decode batches.

This module only draws inputs: context lengths, a permutation of physical
block ids, and N(0, 1) query/key/value data.  It holds none of the decode or
append arithmetic; block tables and slot mappings come from the host
``BlockManager``.  The same arrays feed the HIP library and, in tests, the
CPU oracle, so both sides see identical bits.

Shapes follow the model layers the pages discuss (Habr KV-Cache article,
§2 "KV-Cache: the price of memory": Llama-class layers with 8 KV heads of
dimension 128 and grouped-query attention; §4: 16-token blocks scattered
over the pool; §7: a 2,000-token shared system prompt is 125 blocks;
"Chapter 8 — Next-generation KV cache", §8.1: best-of-8 sampling over one
2,000-token prompt).

Pool layouts: K ``[num_blocks, Hkv, 16, D]``, V ``[num_blocks, Hkv, D, 16]``.
fp8 pools hold OCP E4M3FN codes (uint8) with one float32 scale per kv head;
their initial contents are N(0, 1) bf16 values stored through torch's own
float8 cast after dividing by the per-head scale max|x| / 448, standing in
for a cache that an earlier step filled.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

from .block_manager import BLOCK_SIZE, BlockManager

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class Workload:
    name: str
    kv_dtype: str            # "f32" | "bf16" | "fp8"
    q_dtype: str             # "f32" | "bf16"
    num_blocks: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    q: torch.Tensor          # [B, Hq, D]
    k_pool: torch.Tensor     # [NB, Hkv, 16, D]
    v_pool: torch.Tensor     # [NB, Hkv, D, 16]
    block_tables: torch.Tensor   # int32 [B, max_blocks], -1 past each sequence's blocks
    context_lens: torch.Tensor   # int32 [B]
    scale: float
    k_scale: Optional[torch.Tensor] = None   # float32 [Hkv] (fp8 pools)
    v_scale: Optional[torch.Tensor] = None
    # one decode step's append (None for decode-only workloads)
    k_new: Optional[torch.Tensor] = None     # [T, Hkv, D]
    v_new: Optional[torch.Tensor] = None
    slot_mapping: Optional[torch.Tensor] = None      # int64 [T]
    block_tables_after: Optional[torch.Tensor] = None
    context_lens_after: Optional[torch.Tensor] = None
    unique_blocks: int = 0       # distinct physical blocks the sequences reference

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    def kv_bytes(self, after_append: bool = False) -> int:
        """Bytes of K and V that one decode pass reads (each token once per kv head)."""
        lens = self.context_lens_after if after_append else self.context_lens
        q_bytes = 1 if self.kv_dtype == "fp8" else torch.tensor([], dtype=_TORCH_DTYPE[self.kv_dtype]).element_size()
        return int(lens.to(torch.int64).sum()) * 2 * self.num_kv_heads * self.head_dim * q_bytes


def _randn(shape, gen: torch.Generator, dtype: torch.dtype, chunk_rows: int = 4096) -> torch.Tensor:
    """N(0, 1) drawn in float32 then rounded to ``dtype``, in row chunks to bound memory."""
    out = torch.empty(shape, dtype=dtype)
    rows = shape[0]
    for lo in range(0, rows, chunk_rows):
        hi = min(rows, lo + chunk_rows)
        out[lo:hi] = torch.randn((hi - lo,) + tuple(shape[1:]), generator=gen, dtype=torch.float32).to(dtype)
    return out


def _fp8_pool(shape, gen: torch.Generator, head_axis: int = 1):
    """E4M3 codes and per-head scales standing in for an already-filled fp8 cache."""
    x = _randn(shape, gen, torch.bfloat16)
    num_heads = shape[head_axis]
    amax = torch.stack([x.select(head_axis, h).float().abs().max() for h in range(num_heads)])
    scale = (amax / 448.0).to(torch.float32)
    codes = torch.empty(shape, dtype=torch.uint8)
    for h in range(num_heads):
        xs = x.select(head_axis, h).float() / scale[h]
        codes.select(head_axis, h).copy_(xs.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8))
    return codes, scale


def build_workload(name: str, context_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                   head_dim: int, kv_dtype: str, seed: int, *, shared_prefix: int = 0,
                   with_append: bool = False, num_blocks: Optional[int] = None,
                   max_blocks: Optional[int] = None,
                   rng: Optional[np.random.Generator] = None, block_size: int = BLOCK_SIZE) -> Workload:
    """Seeded workload: pool, tables and queries for one decode step of one layer.

    ``shared_prefix`` tokens (a multiple of the block size) are held once, in
    refcounted blocks that every sequence's table points at.  ``with_append``
    also draws one new token per sequence and reserves its slot.
    """
    BS = int(block_size)
    rng = np.random.default_rng(seed) if rng is None else rng
    gen = torch.Generator().manual_seed(seed)
    lens = [int(n) for n in context_lens]
    B = len(lens)
    if shared_prefix % BS:
        raise ValueError("shared prefix must end on a block boundary")
    if any(n < shared_prefix for n in lens):
        raise ValueError("every sequence must hold the whole shared prefix")

    def nblk(n):
        return (n + BS - 1) // BS

    prefix_blocks = shared_prefix // BS
    needed = prefix_blocks + sum(nblk(n) - prefix_blocks for n in lens)
    if with_append:
        needed += sum(1 for n in lens if n % BS == 0)
    NB = needed + B if num_blocks is None else int(num_blocks)
    if NB < needed:
        raise ValueError(f"pool of {NB} blocks cannot hold {needed}")

    bm = BlockManager(NB, free_order=rng.permutation(NB), block_size=BS)
    if shared_prefix:
        root = bm.new_sequence(shared_prefix)
        ids = []
        for n in lens:
            sid = bm.fork(root)
            bm.extend(sid, n - shared_prefix)
            ids.append(sid)
        bm.free_sequence(root)
    else:
        ids = [bm.new_sequence(n) for n in lens]

    lens_after = [n + 1 for n in lens] if with_append else lens
    width = max(1, max(nblk(n) for n in lens_after)) if max_blocks is None else int(max_blocks)
    tables = bm.block_table(ids, width)
    unique = bm.blocks_in_use()

    D, Hkv, Hq = head_dim, num_kv_heads, num_q_heads
    q_dtype = "f32" if kv_dtype == "f32" else "bf16"
    q = _randn((B, Hq, D), gen, _TORCH_DTYPE[q_dtype])
    k_scale = v_scale = None
    if kv_dtype == "fp8":
        k_pool, k_scale = _fp8_pool((NB, Hkv, BS, D), gen)
        v_pool, v_scale = _fp8_pool((NB, Hkv, D, BS), gen)
    else:
        k_pool = _randn((NB, Hkv, BS, D), gen, _TORCH_DTYPE[kv_dtype])
        v_pool = _randn((NB, Hkv, D, BS), gen, _TORCH_DTYPE[kv_dtype])

    wl = Workload(name=name, kv_dtype=kv_dtype, q_dtype=q_dtype, num_blocks=NB,
                  num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D, q=q,
                  k_pool=k_pool, v_pool=v_pool,
                  block_tables=torch.from_numpy(tables),
                  context_lens=torch.tensor(lens, dtype=torch.int32),
                  scale=float(np.float32(1.0 / math.sqrt(D))),
                  k_scale=k_scale, v_scale=v_scale, unique_blocks=unique)
    if with_append:
        new_dtype = torch.bfloat16 if kv_dtype == "fp8" else _TORCH_DTYPE[kv_dtype]
        wl.k_new = _randn((B, Hkv, D), gen, new_dtype)
        wl.v_new = _randn((B, Hkv, D), gen, new_dtype)
        wl.slot_mapping = torch.tensor([bm.append_slot(s) for s in ids], dtype=torch.int64)
        wl.block_tables_after = torch.from_numpy(bm.block_table(ids, width))
        wl.context_lens_after = torch.tensor(lens_after, dtype=torch.int32)
        wl.unique_blocks = bm.blocks_in_use()
    return wl


# ---------------------------------------------------------------------------
# The five workload shapes
# ---------------------------------------------------------------------------
def tiny_fp32(seed: int = 1, block_size: int = BLOCK_SIZE) -> Workload:
    """4 sequences of 17/33/50/64 tokens, 4 q / 2 kv heads, D 64, fp32, 32-block
    pool in seeded random order, plus one appended token per sequence."""
    return build_workload("tiny-fp32", [17, 33, 50, 64], 4, 2, 64, "f32", seed,
                          with_append=True, num_blocks=32 if block_size == BLOCK_SIZE else None,
                          block_size=block_size)


def llama8b_b64(seed: int = 2, block_size: int = BLOCK_SIZE) -> Workload:
    """Llama-3-8B-shaped layer: batch 64, 32 q / 8 kv heads, D 128, bf16,
    context lengths uniform in [512, 4096], shuffled pool."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(512, 4097, size=64)
    return build_workload("llama3-8b-b64", lens, 32, 8, 128, "bf16", seed, rng=rng, block_size=block_size)


def llama70b_long(seed: int = 3, block_size: int = BLOCK_SIZE) -> Workload:
    """Llama-3-70B-shaped layer, long context: batch 8, 64 q / 8 kv heads, D 128,
    bf16, context lengths uniform in [32768, 131072]."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(32768, 131073, size=8)
    return build_workload("llama3-70b-long", lens, 64, 8, 128, "bf16", seed, rng=rng, block_size=block_size)


def shared_prefix_256(seed: int = 4, block_size: int = BLOCK_SIZE) -> Workload:
    """256 sequences sharing one 4096-token prefix (256 refcounted blocks) plus
    private tails of 64..512 tokens; 32 q / 8 kv heads, D 128, bf16."""
    rng = np.random.default_rng(seed)
    lens = 4096 + rng.integers(64, 513, size=256)
    return build_workload("shared-prefix-256", lens, 32, 8, 128, "bf16", seed,
                          shared_prefix=4096, rng=rng, block_size=block_size)


def best_of_8(seed: int = 40, block_size: int = BLOCK_SIZE) -> Workload:
    """Best-of-8 over a 2000-token prompt (125 shared blocks) with divergent
    1..200-token tails; 32 q / 8 kv heads, D 128, bf16."""
    rng = np.random.default_rng(seed)
    lens = 2000 + rng.integers(1, 201, size=8)
    return build_workload("best-of-8", lens, 32, 8, 128, "bf16", seed,
                          shared_prefix=2000, rng=rng, block_size=block_size)


def fp8_b256(seed: int = 5, block_size: int = BLOCK_SIZE) -> Workload:
    """fp8 (E4M3) cache with per-head scales: batch 256, context lengths
    log-uniform in [128, 8192], 32 q / 8 kv heads, D 128, bf16 queries, plus
    one appended bf16 token per sequence."""
    rng = np.random.default_rng(seed)
    lens = np.rint(np.exp(rng.uniform(math.log(128), math.log(8192), size=256))).astype(np.int64)
    return build_workload("fp8-b256", lens, 32, 8, 128, "fp8", seed, with_append=True, rng=rng,
                          block_size=block_size)


@dataclass
class PrefillStep:
    """One chunk of a chunked prefill: the cache after the chunk's tokens were
    appended (``wl``, one sequence of n tokens) and the chunk's queries
    ``q`` ``[1, L, Hq, D]``; query token i sits at position n - L + i."""
    wl: Workload
    q: torch.Tensor

    def flops(self) -> int:
        """Multiply-adds of QK^T and PV, counted as 2 flops each, over the
        tokens every query token sees (causal): 4 * Hq * D per (query, key)."""
        n, L = int(self.wl.context_lens[0]), int(self.q.shape[1])
        seen = sum(max(0, n - L + 1 + i) for i in range(L))
        return 4 * self.wl.num_q_heads * self.wl.head_dim * seen


def prefill_chunks(seed: int = 6, prompt_tokens: int = 10000, chunk: int = 2048, num_q_heads: int = 64,
                   num_kv_heads: int = 8, head_dim: int = 128, kv_dtype: str = "bf16",
                   block_size: int = BLOCK_SIZE) -> List[PrefillStep]:
    """Habr article section 6, "Chunked Prefill": a 10,000-token prompt under a
    2048-token step budget is prefilled in chunks of 2048, 2048, 2048, 2048 and
    1808 tokens, each attending to every chunk before it.  Layer shape of the
    section's model (Llama-3-70B: 64 q / 8 kv heads, D 128), bf16.  One pool
    holds the whole prompt in shuffled 16-token blocks; step k's cache is its
    first n_k tokens (the chunks appended so far)."""
    wl = build_workload("prefill-70b-10k", [prompt_tokens], num_q_heads, num_kv_heads, head_dim, kv_dtype, seed,
                        block_size=block_size)
    gen = torch.Generator().manual_seed(seed + 1000)
    qd = _TORCH_DTYPE["f32" if kv_dtype == "f32" else "bf16"]
    steps = []
    for lo in range(0, prompt_tokens, chunk):
        hi = min(prompt_tokens, lo + chunk)
        part = Workload(**{**wl.__dict__, "context_lens": torch.tensor([hi], dtype=torch.int32)})
        steps.append(PrefillStep(part, _randn((1, hi - lo, num_q_heads, head_dim), gen, qd)))
    return steps


@dataclass
class CowStep:
    """One decode step of a parallel-sampling batch: block copies to make
    first, then one new token per sample written to its slot."""
    copy_src: torch.Tensor      # int32 [C] blocks to copy from (shared originals)
    copy_dst: torch.Tensor      # int32 [C] fresh private blocks
    slot_mapping: torch.Tensor  # int64 [S]
    k_new: torch.Tensor         # [S, Hkv, D] (bf16 for an fp8 pool)
    v_new: torch.Tensor


@dataclass
class CowScenario:
    """Parallel sampling over one prompt whose last block is partly filled:
    every sample forks the whole prompt, so that block is shared and each
    sample copies it before its first token lands there (copy-on-write)."""
    name: str
    kv_dtype: str
    q_dtype: str
    num_blocks: int
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    k_pool: torch.Tensor          # before any step
    v_pool: torch.Tensor
    k_scale: Optional[torch.Tensor]
    v_scale: Optional[torch.Tensor]
    steps: List[CowStep]
    q: torch.Tensor               # [1 + S, Hq, D]: the prompt's own query, then the samples'
    block_tables: torch.Tensor    # int32 [1 + S, max_blocks] after the last step
    context_lens: torch.Tensor    # int32 [1 + S] after the last step
    scale: float
    prompt_blocks: List[int]      # the prompt's physical blocks (never written)


def cow_sampling(name: str, prompt_tokens: int, samples: int, new_tokens: int, num_q_heads: int,
                 num_kv_heads: int, head_dim: int, kv_dtype: str, seed: int) -> CowScenario:
    """Seeded parallel-sampling batch (Habr article §4, "Copy-on-Write for
    parallel sampling"): one prompt of ``prompt_tokens`` tokens, ``samples``
    forks of it, each appending ``new_tokens`` tokens one step at a time."""
    if prompt_tokens % BLOCK_SIZE == 0:
        raise ValueError("the prompt must end inside a block for copy-on-write to occur")
    rng = np.random.default_rng(seed)
    gen = torch.Generator().manual_seed(seed)
    nblk = (prompt_tokens + BLOCK_SIZE - 1) // BLOCK_SIZE
    extra = samples * (1 + (BLOCK_SIZE - 1 + new_tokens) // BLOCK_SIZE)
    NB = nblk + extra + 4
    bm = BlockManager(NB, free_order=rng.permutation(NB))
    root = bm.new_sequence(prompt_tokens)
    prompt_blocks = bm.blocks(root)
    kids = [bm.fork(root) for _ in range(samples)]
    D, Hkv, Hq = head_dim, num_kv_heads, num_q_heads
    q_dtype = "f32" if kv_dtype == "f32" else "bf16"
    new_dtype = _TORCH_DTYPE["bf16" if kv_dtype == "fp8" else kv_dtype]
    k_scale = v_scale = None
    if kv_dtype == "fp8":
        k_pool, k_scale = _fp8_pool((NB, Hkv, BLOCK_SIZE, D), gen)
        v_pool, v_scale = _fp8_pool((NB, Hkv, D, BLOCK_SIZE), gen)
    else:
        k_pool = _randn((NB, Hkv, BLOCK_SIZE, D), gen, _TORCH_DTYPE[kv_dtype])
        v_pool = _randn((NB, Hkv, D, BLOCK_SIZE), gen, _TORCH_DTYPE[kv_dtype])
    steps = []
    for _ in range(new_tokens):
        src, dst, slots = [], [], []
        for sid in kids:
            slot, copy = bm.append_slot_cow(sid)
            if copy is not None:
                src.append(copy[0])
                dst.append(copy[1])
            slots.append(slot)
        steps.append(CowStep(copy_src=torch.tensor(src, dtype=torch.int32),
                             copy_dst=torch.tensor(dst, dtype=torch.int32),
                             slot_mapping=torch.tensor(slots, dtype=torch.int64),
                             k_new=_randn((samples, Hkv, D), gen, new_dtype),
                             v_new=_randn((samples, Hkv, D), gen, new_dtype)))
    ids = [root] + kids
    width = max(len(bm.blocks(s)) for s in ids)
    return CowScenario(name=name, kv_dtype=kv_dtype, q_dtype=q_dtype, num_blocks=NB, num_kv_heads=Hkv,
                       num_q_heads=Hq, head_dim=D, k_pool=k_pool, v_pool=v_pool, k_scale=k_scale,
                       v_scale=v_scale, steps=steps, q=_randn((1 + samples, Hq, D), gen, _TORCH_DTYPE[q_dtype]),
                       block_tables=torch.from_numpy(bm.block_table(ids, width)),
                       context_lens=torch.from_numpy(bm.context_lens(ids)), scale=1.0 / math.sqrt(D),
                       prompt_blocks=prompt_blocks)


WORKLOADS = {
    "tiny-fp32": tiny_fp32,
    "llama3-8b-b64": llama8b_b64,
    "llama3-70b-long": llama70b_long,
    "shared-prefix-256": shared_prefix_256,
    "best-of-8": best_of_8,
    "fp8-b256": fp8_b256,
}


def storage_numpy(t: torch.Tensor) -> np.ndarray:
    """Host array holding a CPU tensor's bits: float32, uint16 (bf16) or uint8."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
