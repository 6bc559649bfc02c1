"""ctypes binding of ``libpkv.so``: argument marshalling only.

Each function checks that the torch tensors match the C ABI's layout
(device, dtype, shape, contiguity), passes their device pointers and the
current HIP stream, and raises on a non-zero status.  Every step of the
computation runs in the library's HIP kernels; there is no fallback path.
Shapes and the cache layout are documented in ``include/pkv.h``:

* q, out   ``[B, Hq, D]``            float32 or bfloat16
* k_pool   ``[NB, Hkv, B, D]``       float32, bfloat16 or uint8 (E4M3 codes)
* v_pool   ``[NB, Hkv, D, B]``       B tokens per block: 16, 32, 64, 128 or 256
* block_tables ``[B, max_blocks]`` int32, context_lens ``[B]`` int32
* slot_mapping ``[T]`` int64; k_new / v_new ``[T, Hkv, D]``
* copy src / dst ``[P]`` int32 block ids
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .build import LIB_PATH

F32, BF16, FP8_E4M3 = 0, 1, 2
BLOCK_SIZE = 16

_lib = None


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("flags", ctypes.c_uint32),
    ]


KV_REREAD = 1   # blocks shared within the batch: keep K/V cached (a hint; same result)


def library() -> ctypes.CDLL:
    """Load ``libpkv.so`` once; a missing library is an error, never a fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        D = ctypes.POINTER(CacheDesc)
        sigs = {
            "pkv_kv_append": (ctypes.c_int, [D, P, P, P, I32, P, P, P]),
            "pkv_copy_blocks": (ctypes.c_int, [D, P, P, P, P, I32, P]),
            "pkv_decode_workers": (I32, [D, I32, I32]),
            "pkv_decode_workspace_bytes": (SZ, [D, I32, I32, I32]),
            "pkv_paged_decode": (ctypes.c_int, [D, P, P, P, P, I32, P, I32, I32, F, P, P, SZ, P]),
            "pkv_paged_decode_ex": (ctypes.c_int, [D, P, P, P, P, I32, P, I32, I32, F, I32, P, P, SZ, P]),
            "pkv_paged_decode_static": (ctypes.c_int, [D, P, P, P, P, I32, P, I32, I32, F, P, P]),
            "pkv_paged_attention": (ctypes.c_int, [D, P, P, P, P, I32, P, I32, I32, I32, F, I32, P, P, SZ, P]),
            "pkv_attention_workspace_bytes": (SZ, [D, I32, I32, I32, I32]),
            "pkv_shared_decode_workspace_bytes": (SZ, [D, I32, I32, I32, I32]),
            "pkv_shared_prefix_pays": (I32, [D, I32, I32]),
            "pkv_paged_decode_shared": (ctypes.c_int,
                                        [D, P, P, P, P, I32, P, I32, I32, I32, F, I32, P, P, SZ, P]),
            "pkv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
            "pkv_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        raise RuntimeError(f"{what}: {library().pkv_strerror(status).decode()} (status {status})")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require(t: torch.Tensor, name: str, dtypes, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _kv_code(pool: torch.Tensor) -> int:
    if pool.dtype == torch.float32:
        return F32
    if pool.dtype == torch.bfloat16:
        return BF16
    if pool.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise ValueError(f"unsupported cache dtype {pool.dtype}")


def cache_desc(k_pool: torch.Tensor, v_pool: torch.Tensor, num_q_heads: int,
               k_scale: Optional[torch.Tensor] = None,
               v_scale: Optional[torch.Tensor] = None, reread: bool = False) -> CacheDesc:
    """Descriptor for pools ``k_pool [NB, Hkv, B, D]`` / ``v_pool [NB, Hkv, D, B]``."""
    kv = _kv_code(k_pool)
    _require(k_pool, "k_pool", (k_pool.dtype,), 4)
    _require(v_pool, "v_pool", (k_pool.dtype,), 4)
    NB, Hkv, bs, D = k_pool.shape
    if tuple(v_pool.shape) != (NB, Hkv, D, bs):
        raise ValueError(f"pool shapes {tuple(k_pool.shape)} / {tuple(v_pool.shape)} do not match "
                         "[NB, Hkv, B, D] / [NB, Hkv, D, B]")
    if kv == FP8_E4M3:
        if k_scale is None or v_scale is None:
            raise ValueError("an fp8 cache needs k_scale and v_scale")
        for name, sc in (("k_scale", k_scale), ("v_scale", v_scale)):
            _require(sc, name, (torch.float32,), 1)
            if sc.shape[0] != Hkv:
                raise ValueError(f"{name} must have {Hkv} entries")
    elif k_scale is not None or v_scale is not None:
        raise ValueError("scales are only used with an fp8 cache")
    return CacheDesc(NB, bs, Hkv, int(num_q_heads), D, kv,
                     F32 if kv == F32 else BF16, _ptr(k_scale), _ptr(v_scale), KV_REREAD if reread else 0)


def kv_append(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
              k_pool: torch.Tensor, v_pool: torch.Tensor, k_scale: Optional[torch.Tensor] = None,
              v_scale: Optional[torch.Tensor] = None, stream=None) -> None:
    """Write each token's K/V ``[T, Hkv, D]`` into slot ``slot_mapping[t]`` of the pools (in place)."""
    Hkv = k_pool.shape[1]
    desc = cache_desc(k_pool, v_pool, Hkv, k_scale, v_scale)
    new_dtype = torch.bfloat16 if desc.kv_dtype == FP8_E4M3 else k_pool.dtype
    _require(k_new, "k_new", (new_dtype,), 3)
    _require(v_new, "v_new", (new_dtype,), 3)
    _require(slot_mapping, "slot_mapping", (torch.int64,), 1)
    T = slot_mapping.shape[0]
    if tuple(k_new.shape) != (T, Hkv, desc.head_dim) or k_new.shape != v_new.shape:
        raise ValueError(f"k_new/v_new must be [{T}, {Hkv}, {desc.head_dim}]")
    _check(library().pkv_kv_append(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                                   T, _ptr(k_pool), _ptr(v_pool), _stream(stream)), "pkv_kv_append")


def copy_blocks(k_pool: torch.Tensor, v_pool: torch.Tensor, src: torch.Tensor, dst: torch.Tensor,
                k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """Copy block ``src[i]`` to block ``dst[i]`` in both pools (copy-on-write), in place."""
    desc = cache_desc(k_pool, v_pool, k_pool.shape[1], k_scale, v_scale)
    _require(src, "src", (torch.int32,), 1)
    _require(dst, "dst", (torch.int32,), 1)
    if src.shape != dst.shape:
        raise ValueError("src and dst must have the same length")
    _check(library().pkv_copy_blocks(ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool), _ptr(src), _ptr(dst),
                                     src.shape[0], _stream(stream)), "pkv_copy_blocks")


def _decode_checks(q, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, out, reread=False):
    desc = cache_desc(k_pool, v_pool, q.shape[1] if q.dim() == 3 else 0, k_scale, v_scale, reread)
    q_dtype = torch.float32 if desc.q_dtype == F32 else torch.bfloat16
    _require(q, "q", (q_dtype,), 3)
    B = q.shape[0]
    if q.shape[2] != desc.head_dim:
        raise ValueError(f"q head_dim {q.shape[2]} != cache head_dim {desc.head_dim}")
    _require(block_tables, "block_tables", (torch.int32,), 2)
    _require(context_lens, "context_lens", (torch.int32,), 1)
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", (q_dtype,), 3)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    return desc, out


def _max_ctx(block_tables: torch.Tensor, max_context_len: Optional[int], block_size: int = BLOCK_SIZE) -> int:
    # without a host-side value, the table width bounds every length (no device sync)
    return int(max_context_len) if max_context_len is not None else block_size * block_tables.shape[1]


def decode_workers(k_pool, v_pool, num_q_heads: int, num_seqs: int, max_context_len: int,
                   k_scale=None, v_scale=None) -> int:
    """Worker waves the decode uses for this shape on the current device."""
    desc = cache_desc(k_pool, v_pool, num_q_heads, k_scale, v_scale)
    res = library().pkv_decode_workers(ctypes.byref(desc), num_seqs, max_context_len)
    _check(min(res, 0), "pkv_decode_workers")
    return res


def decode_workspace_bytes(k_pool, v_pool, num_q_heads: int, num_seqs: int, max_context_len: int,
                           num_workers: int = 0, k_scale=None, v_scale=None) -> int:
    desc = cache_desc(k_pool, v_pool, num_q_heads, k_scale, v_scale)
    return int(library().pkv_decode_workspace_bytes(ctypes.byref(desc), num_seqs, max_context_len, num_workers))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A decode workspace (scratch; reusable by calls ordered on one stream)."""
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _temp_workspace(nbytes: int, device, stream) -> torch.Tensor:
    """Scratch for one call.  It is freed when the call returns, while the
    kernels may still be queued, so it is allocated on the stream they run
    on: torch's caching allocator then reuses it only for later work on that
    same stream, which runs after them."""
    if stream is None:
        return new_workspace(nbytes, device)
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)), device=device)
    with torch.cuda.stream(stream):
        return new_workspace(nbytes, device)


def attention_workspace_bytes(k_pool, v_pool, num_q_heads: int, num_seqs: int, q_len: int,
                              max_context_len: int, num_workers: int = 0, k_scale=None, v_scale=None) -> int:
    desc = cache_desc(k_pool, v_pool, num_q_heads, k_scale, v_scale)
    return int(library().pkv_attention_workspace_bytes(ctypes.byref(desc), num_seqs, q_len, max_context_len,
                                                       num_workers))


def paged_attention(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                    block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                    out: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
                    v_scale: Optional[torch.Tensor] = None, max_context_len: Optional[int] = None,
                    workspace: Optional[torch.Tensor] = None, num_workers: int = 0,
                    stream=None, reread: bool = False) -> torch.Tensor:
    """Causal attention of the last ``L`` tokens of each sequence: q and out ``[B, L, Hq, D]``.

    Up to 16 (query token, head) columns per kv head run on the split decode
    kernels (speculative verification); more run on the prefill kernel
    (chunked prefill), which needs no workspace.  ``reread``: the tables
    share blocks (see ``paged_decode``)."""
    _require(q, "q", (torch.float32, torch.bfloat16), 4)
    B, L, Hq, D = q.shape
    desc, _ = _decode_checks(q.view(B, L * Hq, D), k_pool, v_pool, block_tables, context_lens, k_scale, v_scale,
                             None, reread)
    desc.num_q_heads = Hq
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", (q.dtype,), 4)
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    mctx = _max_ctx(block_tables, max_context_len, k_pool.shape[2])
    lib = library()
    need = lib.pkv_attention_workspace_bytes(ctypes.byref(desc), B, L, mctx, int(num_workers))
    if need == 0 and B > 0:
        _check(-2 if L * (Hq // desc.num_kv_heads) > 1 << 24 else -1, "pkv_attention_workspace_bytes")
    if workspace is None:
        workspace = _temp_workspace(need, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size()
    if workspace.device.type != "cuda" or wbytes < need:
        raise ValueError(f"workspace must be a device buffer of at least {need} bytes")
    _check(lib.pkv_paged_attention(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                   block_tables.shape[1], _ptr(context_lens), B, L, mctx, float(scale),
                                   int(num_workers), _ptr(out), _ptr(workspace), wbytes, _stream(stream)),
           "pkv_paged_attention")
    return out


def paged_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                 block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                 out: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
                 v_scale: Optional[torch.Tensor] = None, max_context_len: Optional[int] = None,
                 workspace: Optional[torch.Tensor] = None, num_workers: int = 0,
                 stream=None, reread: bool = False) -> torch.Tensor:
    """Decode attention of one query per sequence over its paged K/V; returns ``out``.

    ``reread``: the tables share blocks between sequences (prefix sharing,
    parallel sampling), so K/V are loaded cached instead of streamed; a speed
    hint only, the result is the same.

    ``workspace`` (optional) must hold ``decode_workspace_bytes`` bytes for the
    same shape and ``num_workers``; calls sharing it must run on one stream.
    """
    desc, out = _decode_checks(q, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, out, reread)
    mctx = _max_ctx(block_tables, max_context_len, k_pool.shape[2])
    lib = library()
    need = lib.pkv_decode_workspace_bytes(ctypes.byref(desc), q.shape[0], mctx, int(num_workers))
    if need == 0 and q.shape[0] > 0:
        _check(-1, "pkv_decode_workspace_bytes")
    if workspace is None:
        workspace = _temp_workspace(need, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size()
    if workspace.device.type != "cuda" or wbytes < need:
        raise ValueError(f"workspace must be a device buffer of at least {need} bytes")
    _check(lib.pkv_paged_decode_ex(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                   block_tables.shape[1], _ptr(context_lens), q.shape[0], mctx, float(scale),
                                   int(num_workers), _ptr(out), _ptr(workspace), wbytes, _stream(stream)),
           "pkv_paged_decode_ex")
    return out


STATIC_SCRATCH_BYTES = 32 << 20   # the library's static decode workspace per device


def paged_decode_static(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                        block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                        out: torch.Tensor, k_scale: Optional[torch.Tensor] = None,
                        v_scale: Optional[torch.Tensor] = None, max_context_len: Optional[int] = None,
                        stream=None, reread: bool = False) -> torch.Tensor:
    """``paged_decode`` that allocates nothing: the caller passes ``out`` and the
    library uses its own static device workspace (``STATIC_SCRATCH_BYTES`` per
    device; larger batches raise).  Calls that overlap on one device race."""
    desc, out = _decode_checks(q, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, out, reread)
    mctx = _max_ctx(block_tables, max_context_len, k_pool.shape[2])
    _check(library().pkv_paged_decode_static(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                             _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                             q.shape[0], mctx, float(scale), _ptr(out), _stream(stream)),
           "pkv_paged_decode_static")
    return out


def shared_decode_workspace_bytes(k_pool, v_pool, num_q_heads: int, num_seqs: int, max_context_len: int,
                                  prefix_tokens: int, num_workers: int = 0, k_scale=None, v_scale=None) -> int:
    desc = cache_desc(k_pool, v_pool, num_q_heads, k_scale, v_scale)
    return int(library().pkv_shared_decode_workspace_bytes(ctypes.byref(desc), num_seqs, max_context_len,
                                                           prefix_tokens, num_workers))


def paged_decode_shared(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                        block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                        prefix_tokens: int, out: Optional[torch.Tensor] = None,
                        k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                        max_context_len: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                        num_workers: int = 0, stream=None, always: bool = True) -> torch.Tensor:
    """``paged_decode`` for a batch whose table rows all start with the same
    ``prefix_tokens // block_size`` blocks (parallel sampling over one prompt).

    The prefix's K/V are read once for the whole batch.  ``prefix_tokens`` is
    a multiple of the block size and every sequence holds at least that many
    tokens; ``workspace`` must hold ``shared_decode_workspace_bytes`` bytes.
    ``always=False`` runs the plain decode (cached loads) instead when
    ``shared_prefix_pays`` says the batch is too small to gain.
    """
    desc, out = _decode_checks(q, k_pool, v_pool, block_tables, context_lens, k_scale, v_scale, out, False)
    mctx = _max_ctx(block_tables, max_context_len, k_pool.shape[2])
    lib = library()
    B = q.shape[0]
    if not always:
        pays = lib.pkv_shared_prefix_pays(ctypes.byref(desc), B, int(prefix_tokens))
        _check(min(pays, 0), "pkv_shared_prefix_pays")
        if not pays:
            return paged_decode(q, k_pool, v_pool, block_tables, context_lens, scale, out=out, k_scale=k_scale,
                                v_scale=v_scale, max_context_len=max_context_len, num_workers=num_workers,
                                stream=stream, reread=True)
    need = lib.pkv_shared_decode_workspace_bytes(ctypes.byref(desc), B, mctx, int(prefix_tokens), int(num_workers))
    if need == 0:
        _check(-1, "pkv_shared_decode_workspace_bytes")
    if workspace is None:
        workspace = _temp_workspace(need, q.device, stream)
    wbytes = workspace.numel() * workspace.element_size()
    if workspace.device.type != "cuda" or wbytes < need:
        raise ValueError(f"workspace must be a device buffer of at least {need} bytes")
    _check(lib.pkv_paged_decode_shared(ctypes.byref(desc), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                       block_tables.shape[1], _ptr(context_lens), B, mctx, int(prefix_tokens),
                                       float(scale), int(num_workers), _ptr(out), _ptr(workspace), wbytes,
                                       _stream(stream)),
           "pkv_paged_decode_shared")
    return out


def shared_prefix_pays(k_pool, v_pool, num_q_heads: int, num_seqs: int, prefix_tokens: int,
                       k_scale=None, v_scale=None) -> bool:
    """Whether the shared-prefix decode is expected to beat the plain one."""
    desc = cache_desc(k_pool, v_pool, num_q_heads, k_scale, v_scale)
    res = library().pkv_shared_prefix_pays(ctypes.byref(desc), num_seqs, prefix_tokens)
    _check(min(res, 0), "pkv_shared_prefix_pays")
    return bool(res)
