"""Plain fp64 oracle for the paged KV cache: append and decode attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources (all readings are the plainest the pages support):

* Habr KV-Cache article (habr.com/ru/articles/1021832), §3 "Recalling
  FlashAttention": attention is softmax(Q K^T / sqrt(d_k)) V; the tiled
  online-softmax form reaches the same result with no approximation, so
  this oracle is that plain definition, evaluated per decode query.
* Same article, §4 "Recalling PagedAttention", subsection "Blocks and block
  table": the cache is cut into fixed 16-token blocks that need not be
  contiguous; a per-sequence block table maps logical block j to a
  physical block id.  §5 "How vLLM combines FlashAttention and
  PagedAttention", code sample: the decode call takes one query per
  sequence, the K/V caches, an int32 table [batch, max_num_blocks] and the
  true length of each sequence.
* "Chapter 8 — Next-generation KV cache" (LLM Primer VI), §8.1: the
  kernel gathers keys and values through the table by indirect addressing
  instead of a contiguous slice.  This oracle makes the gather explicit:
  it copies each sequence's blocks into a contiguous slab first.
* Same Habr article, §1 "Prefill and Decode": each decode step appends the
  new token's K and V to the cache.

Layout reading (the pages print a third-party API's layout only; this
library stores tiles so that one (block, kv-head) tile is contiguous):

* K pool: ``[num_blocks, num_kv_heads, B, head_dim]``  (token-major tile)
* V pool: ``[num_blocks, num_kv_heads, head_dim, B]``  (dim-major tile)
* B tokens per block, 16 by default (taken from the pool's shape);
* slot s (int64) names block ``s // B`` and offset ``s % B``; a slot
  outside ``[0, num_blocks * B)`` is padding and writes nothing.

Storage dtypes are given by name: ``"f32"`` (float32 arrays), ``"bf16"``
(uint16 arrays holding the bf16 bit patterns) and ``"fp8"`` (uint8 arrays
holding OCP E4M3FN codes, with per-kv-head float32 scales).
"""

from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16  # default tokens per block: Habr article §4, "Blocks and block table"


def block_size_of(k_pool) -> int:
    """Tokens per block of a K pool ``[num_blocks, Hkv, block_size, D]``.

    Habr article §4, "Choosing the block size": 16 is the default; larger
    blocks (up to 256 in the page's table) trade internal fragmentation for a
    smaller block table.  Every function here takes the block size from the
    pools it is given.
    """
    return int(np.shape(k_pool)[2])


# --------------------------------------------------------------------------
# Closed form for the cache size
# --------------------------------------------------------------------------
def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """Bytes of K and V one token occupies: 2 x L x Hkv x D x q.

    Habr article §2 "KV-Cache: the price of memory" (formula), repeated in
    "Why one character breaks the cache" (section on why the cache is
    expensive to store) and in "Shared KV-cache across replicas without
    self-deception" (section on counting KV size by KV heads).  The factor 2
    is one K and one V; the head count is the KV head count, not the query
    head count.
    """
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 is the upper half of an IEEE binary32 word, so widening is exact."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        return u.view(np.float32).astype(np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """Value of OCP E4M3FN codes (the 8-bit float named by the fp8 KV option).

    Habr article §2 names an fp8 KV cache (half the bytes per token);
    "Shared KV-cache across replicas", section on KV size, says the exact
    format comes from the engine's configuration.  The reading here is OCP
    E4M3FN: sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
    field 0 holds subnormals m/8 * 2^-6; S.1111.111 is NaN; no infinities.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def e4m3_encode(x) -> np.ndarray:
    """Round float32 values to OCP E4M3FN codes: nearest, ties to even, saturating.

    Reading of the fp8 cache format (see ``e4m3_decode``): magnitudes at or
    above the largest finite value 448 (including infinities) become +-448;
    NaN becomes the NaN code with the input's sign bit; -0 keeps its sign.
    Within one binade [2^E, 2^(E+1)) the grid spacing is 2^(E-3); below
    2^-6 the subnormal grid keeps the spacing 2^-9 of the lowest binade.
    A value's code is then (E + 7) * 8 + (nearest multiple of the spacing,
    counted in spacings) - 8, which also carries a round-up across a binade
    edge into the next exponent.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    finite = np.isfinite(a)
    a_f = np.where(finite, a, 0.0)
    _, k = np.frexp(a_f)  # a = f * 2^k with f in [0.5, 1)
    binade = np.where(a_f < 2.0 ** -6, -6, k - 1)
    spacing = np.exp2(binade.astype(np.float64) - 3.0)
    steps = np.rint(a_f / spacing)  # exact power-of-two division; rint ties to even
    code = (binade + 7) * 8 + steps.astype(np.int64) - 8
    code = np.where(a >= 448.0, 0x7E, code)  # saturate (infinities included)
    code = np.where(np.isnan(x), 0x7F, code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def _widen(arr, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "fp8":
        return e4m3_decode(arr)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# Append
# --------------------------------------------------------------------------
def oracle_append(k_pool, v_pool, k_new, v_new, slot_mapping, kv_dtype: str,
                  k_scale=None, v_scale=None):
    """Write each new token's K and V into its slot; return new pool copies.

    Habr article §1 "Prefill and Decode": a decode step computes K and V
    for the one new token and appends them to the cache.  §4 worked example:
    the token goes to the next slot of the sequence's last block, opening a
    fresh block when the last one is full (the caller chose the slot).

    ``k_new``/``v_new`` are ``[T, Hkv, D]`` in the pool's dtype for f32/bf16
    (a raw bit copy), or bf16 bits for the fp8 pool, where the stored code is
    e4m3(float32(x) / float32(scale[h])) with IEEE float32 division.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    T = slots.shape[0]
    num_kv_heads = k_out.shape[1]
    bs = block_size_of(k_out)
    num_slots = k_out.shape[0] * bs
    for i in range(T):
        s = int(slots[i])
        if s < 0 or s >= num_slots:
            continue  # padding token: nothing to write
        blk, off = s // bs, s % bs
        for h in range(num_kv_heads):
            if kv_dtype == "fp8":
                kx = bf16_bits_to_f64(k_new[i, h]).astype(np.float32)
                vx = bf16_bits_to_f64(v_new[i, h]).astype(np.float32)
                kc = e4m3_encode(kx / np.float32(k_scale[h]))
                vc = e4m3_encode(vx / np.float32(v_scale[h]))
            else:
                kc, vc = k_new[i, h], v_new[i, h]
            k_out[blk, h, off, :] = kc  # K tile is token-major
            v_out[blk, h, :, off] = vc  # V tile is dim-major
    return k_out, v_out


def oracle_copy_blocks(k_pool, v_pool, src, dst):
    """Copy whole blocks (every kv head, K and V) from src[i] to dst[i].

    Habr article §4, subsection "Copy-on-Write for parallel sampling": when a
    sequence must modify a block that other sequences reference, the block
    is copied first and the original stays untouched; §8 gives the same rule
    for a speculative correction landing in a shared block.  "Why one
    character breaks the cache" (PagedAttention as virtual memory): the
    engine counts references per block and copies at block granularity.

    Pairs whose source or destination lies outside ``[0, num_blocks)`` are
    skipped.  The pairs are applied in order; the library's contract (distinct
    destinations, none of them also a source) makes the order irrelevant.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    nb = k_out.shape[0]
    for s_blk, d_blk in zip(np.asarray(src, dtype=np.int64), np.asarray(dst, dtype=np.int64)):
        if not (0 <= s_blk < nb and 0 <= d_blk < nb):
            continue
        k_out[d_blk] = k_out[s_blk]
        v_out[d_blk] = v_out[s_blk]
    return k_out, v_out


# --------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------
def gather_slab(pool, table_row, n: int, which: str, head: int) -> np.ndarray:
    """Copy the first n tokens of one sequence and one kv head into a slab.

    Logical block j of the sequence lives in physical block
    ``table_row[j]``; with B tokens per block, only blocks j < ceil(n / B)
    are read, and only the first n - B j tokens of the last one.  Returns
    ``[n, D]`` in the pool's storage dtype.
    """
    head_dim = pool.shape[3] if which == "k" else pool.shape[2]
    bs = pool.shape[2] if which == "k" else pool.shape[3]
    slab = np.empty((n, head_dim), dtype=pool.dtype)
    num_blocks = (n + bs - 1) // bs
    for j in range(num_blocks):
        phys = int(table_row[j])
        lo = j * bs
        cnt = min(bs, n - lo)
        if which == "k":
            slab[lo:lo + cnt] = pool[phys, head, :cnt, :]
        else:
            slab[lo:lo + cnt] = pool[phys, head, :, :cnt].T
    return slab


def softmax_weights(scores) -> np.ndarray:
    """Two-pass softmax in fp64: subtract the maximum, exponentiate, normalise."""
    s = np.asarray(scores, dtype=np.float64)
    e = np.exp(s - s.max())
    return e / e.sum()


def _attend_pair(qf_rows, K, V, scale64):
    """Attention of G query rows against one kv head's slab: [G, D]."""
    out = np.empty((qf_rows.shape[0], V.shape[1]))
    for r in range(qf_rows.shape[0]):
        w = softmax_weights(scale64 * (K @ qf_rows[r]))
        out[r] = w @ V
    return out


def oracle_decode_pairs(q, q_dtype: str, k_pool, v_pool, kv_dtype: str,
                        block_tables, context_lens, scale: float, pairs,
                        k_scale=None, v_scale=None) -> np.ndarray:
    """Decode outputs for selected (sequence, kv head) pairs: ``[len(pairs), G, D]``.

    For pair (b, g), the query heads g*G .. g*G+G-1 share kv head g
    (grouped-query attention: Habr article §2, "GQA: 8x reduction", where
    each KV head serves a contiguous group of query heads).  Each head's
    output is softmax(scale * q . K^T) V over the sequence's n tokens,
    evaluated in fp64 on the gathered slab.  The scale is the float32 value
    passed, widened.  A sequence of length 0 yields zeros.  For fp8 pools the
    codes are decoded and multiplied by the kv head's float32 scale.
    """
    q = np.asarray(q)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.zeros((len(pairs), G, D))
    for idx, (b, g) in enumerate(pairs):
        n = int(context_lens[b])
        if n == 0:
            continue
        K = _widen(gather_slab(k_pool, block_tables[b], n, "k", g), kv_dtype)
        V = _widen(gather_slab(v_pool, block_tables[b], n, "v", g), kv_dtype)
        if kv_dtype == "fp8":
            K = K * float(np.float32(k_scale[g]))
            V = V * float(np.float32(v_scale[g]))
        qf = _widen(q[b, g * G:(g + 1) * G], q_dtype)
        out[idx] = _attend_pair(qf, K, V, scale64)
    return out


def oracle_decode(q, q_dtype: str, k_pool, v_pool, kv_dtype: str,
                  block_tables, context_lens, scale: float,
                  k_scale=None, v_scale=None) -> np.ndarray:
    """Full decode output ``[B, Hq, D]`` in fp64 (every pair of ``oracle_decode_pairs``)."""
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    res = oracle_decode_pairs(q, q_dtype, k_pool, v_pool, kv_dtype, block_tables,
                              context_lens, scale, pairs, k_scale, v_scale)
    return res.reshape(B, Hkv * G, D)


# --------------------------------------------------------------------------
# Several query tokens per sequence
# --------------------------------------------------------------------------
def oracle_attention_multi(q, q_dtype: str, k_pool, v_pool, kv_dtype: str,
                           block_tables, context_lens, scale: float,
                           k_scale=None, v_scale=None) -> np.ndarray:
    """Causal attention of the last L tokens of each sequence: ``[B, L, Hq, D]``.

    Habr article §6 "Chunked Prefill": a prompt chunk is processed in one
    forward pass next to decode tokens, attending to everything cached before
    it; "Chapter 8 - Next-generation KV cache", closing section: speculative
    decoding verifies several drafted tokens in one pass.  In both, the L new
    tokens' K and V are already in the cache (appended first, as for decode),
    so sequence b holds n = context_lens[b] >= L tokens and query token i
    (i < L) sits at position n - L + i: it attends to the first n - L + i + 1
    tokens (itself and everything before it; causal attention, Habr §3).
    Each output row is the plain softmax(scale * q . K^T) V over those
    tokens, evaluated in fp64 on the gathered slab; query heads share kv
    heads in contiguous groups as for decode.
    """
    q = np.asarray(q)
    B, L, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.zeros((B, L, Hq, D))
    for b in range(B):
        n = int(context_lens[b])
        if n < L:
            raise ValueError(f"sequence {b} holds {n} tokens, fewer than its {L} query tokens")
        for g in range(Hkv):
            K = _widen(gather_slab(k_pool, block_tables[b], n, "k", g), kv_dtype)
            V = _widen(gather_slab(v_pool, block_tables[b], n, "v", g), kv_dtype)
            if kv_dtype == "fp8":
                K = K * float(np.float32(k_scale[g]))
                V = V * float(np.float32(v_scale[g]))
            for i in range(L):
                visible = n - L + i + 1
                qf = _widen(q[b, i, g * G:(g + 1) * G], q_dtype)
                out[b, i, g * G:(g + 1) * G] = _attend_pair(qf, K[:visible], V[:visible], scale64)
    return out

