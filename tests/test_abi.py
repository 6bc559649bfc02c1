"""The C-ABI library loads, exports every declared entry point, and rejects
bad arguments on the host before any HIP call (no GPU needed)."""

from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from paged_kv_cache_23_amd import ops
from paged_kv_cache_23_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB_PATH), reason="libpkv.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("pkv_kv_append", "pkv_copy_blocks", "pkv_paged_decode", "pkv_paged_decode_ex",
                     "pkv_decode_workspace_bytes", "pkv_decode_workers", "pkv_strerror",
                     "pkv_paged_decode_shared", "pkv_shared_decode_workspace_bytes"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (pkv_\w+)", out))
    assert set(declared_functions()) <= exported


def _desc(**kw):
    d = dict(num_blocks=8, block_size=16, num_kv_heads=2, num_q_heads=8, head_dim=128,
             kv_dtype=ops.BF16, q_dtype=ops.BF16, k_scale=None, v_scale=None)
    d.update(kw)
    return ops.CacheDesc(**d)


EINVAL, EUNSUPPORTED, EWORKSPACE = -1, -2, -3
FAKE = 0x10000  # a non-null, 16-byte aligned address that is never dereferenced


@pytest.mark.parametrize("kw,code", [
    (dict(block_size=48), EINVAL),           # block sizes: 16, 32, 64, 128, 256
    (dict(block_size=8), EINVAL),
    (dict(block_size=512), EINVAL),
    (dict(num_blocks=0), EINVAL),
    (dict(num_q_heads=7), EINVAL),
    (dict(num_q_heads=64), EUNSUPPORTED),   # 32 query heads per kv head
    (dict(head_dim=96), EUNSUPPORTED),
    (dict(kv_dtype=ops.F32), EUNSUPPORTED),  # f32 cache with bf16 queries
    (dict(kv_dtype=ops.FP8_E4M3), EINVAL),   # fp8 without scales
    (dict(kv_dtype=7), EINVAL),
    (dict(k_scale=FAKE), EINVAL),            # scales on a bf16 cache
    (dict(flags=2), EINVAL),                 # unknown flag bit
])
def test_bad_descriptors_are_rejected(kw, code):
    lib = ops.library()
    d = _desc(**kw)
    assert lib.pkv_kv_append(ctypes.byref(d), FAKE, FAKE, FAKE, 1, FAKE, FAKE, None) == code
    assert lib.pkv_paged_decode(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 0.1,
                                FAKE, None, 0, None) == code


def test_null_and_size_errors():
    lib = ops.library()
    d = _desc()
    assert lib.pkv_kv_append(None, FAKE, FAKE, FAKE, 1, FAKE, FAKE, None) == EINVAL
    assert lib.pkv_kv_append(ctypes.byref(d), None, FAKE, FAKE, 1, FAKE, FAKE, None) == EINVAL
    assert lib.pkv_kv_append(ctypes.byref(d), FAKE, FAKE, FAKE, -1, FAKE, FAKE, None) == EINVAL
    assert lib.pkv_kv_append(ctypes.byref(d), FAKE + 8, FAKE, FAKE, 1, FAKE, FAKE, None) == EINVAL   # misaligned k_new
    assert lib.pkv_kv_append(ctypes.byref(d), FAKE, FAKE, FAKE, 1, FAKE, FAKE + 2, None) == EINVAL   # misaligned pool
    assert lib.pkv_kv_append(ctypes.byref(d), None, None, None, 0, None, None, None) == 0  # no-op
    assert lib.pkv_paged_decode(ctypes.byref(d), None, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 0.1,
                                FAKE, None, 0, None) == EINVAL
    assert lib.pkv_paged_decode(ctypes.byref(d), FAKE + 8, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 0.1,
                                FAKE, None, 0, None) == EINVAL          # misaligned q
    assert lib.pkv_paged_decode_ex(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 0.1,
                                      6, FAKE, None, 0, None) == EINVAL    # workers not a multiple of 4
    assert lib.pkv_paged_decode_ex(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 0.1,
                                      -4, FAKE, None, 0, None) == EINVAL   # negative workers


def test_copy_blocks_argument_checks():
    lib = ops.library()
    d = _desc()
    assert lib.pkv_copy_blocks(None, FAKE, FAKE, FAKE, FAKE, 1, None) == EINVAL
    assert lib.pkv_copy_blocks(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, -1, None) == EINVAL
    assert lib.pkv_copy_blocks(ctypes.byref(d), None, FAKE, FAKE, FAKE, 1, None) == EINVAL
    assert lib.pkv_copy_blocks(ctypes.byref(d), FAKE, FAKE, None, FAKE, 1, None) == EINVAL
    assert lib.pkv_copy_blocks(ctypes.byref(d), FAKE + 8, FAKE, FAKE, FAKE, 1, None) == EINVAL   # misaligned pool
    assert lib.pkv_copy_blocks(ctypes.byref(d), None, None, None, None, 0, None) == 0             # no-op
    bad = _desc(head_dim=96)
    assert lib.pkv_copy_blocks(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, 1, None) == EUNSUPPORTED


def test_workspace_sizing_and_check():
    lib = ops.library()
    d = _desc()                                 # 8 q heads / 2 kv heads: group 4, head_dim 128
    # (workers + seqs * kv heads) partial states: acc rows, (max, sum) rows and one
    # counter per pair, each region rounded up to 256 bytes
    rows = (64 + 4 * 2) * 4
    up = lambda n: -(-n // 256) * 256
    need = lib.pkv_decode_workspace_bytes(ctypes.byref(d), 4, 150, 64)
    assert need == up(rows * 128 * 4) + up(rows * 2 * 4) + up(4 * 2 * 4)
    assert lib.pkv_decode_workspace_bytes(ctypes.byref(d), 4, 150, 6) == 0     # bad worker count
    st = lib.pkv_paged_decode_ex(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, 150, 0.1,
                                 64, FAKE, FAKE, need - 1, None)
    assert st == EWORKSPACE
    st = lib.pkv_paged_decode_ex(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, 150, 0.1,
                                 64, FAKE, None, need, None)
    assert st == EWORKSPACE
    # zero sequences: nothing to do, nothing launched
    assert lib.pkv_paged_decode_ex(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 16, FAKE, 0, 150, 0.1,
                                   64, FAKE, None, 0, None) == 0


def test_many_query_sizing():
    """Up to 16 (query token, head) columns per kv head use the split kernels'
    workspace; more run on the prefill kernel, which takes none (a nominal 256
    bytes is reported so that 0 still means bad arguments); beyond 2^24
    columns the call is unsupported."""
    lib = ops.library()
    d = _desc()                                 # group 4
    up = lambda n: -(-n // 256) * 256
    rows = (64 + 4 * 2) * 4 * 4                 # q_len 4: 16 columns
    assert lib.pkv_attention_workspace_bytes(ctypes.byref(d), 4, 4, 150, 64) == \
        up(rows * 128 * 4) + up(rows * 2 * 4) + up(4 * 2 * 4)
    assert lib.pkv_attention_workspace_bytes(ctypes.byref(d), 4, 5, 150, 64) == 256
    assert lib.pkv_attention_workspace_bytes(ctypes.byref(d), 4, 2048, 10000, 0) in (0, 256)  # 0 without a GPU
    assert lib.pkv_attention_workspace_bytes(ctypes.byref(d), 4, 1 << 22, 150, 64) == 256
    assert lib.pkv_attention_workspace_bytes(ctypes.byref(d), 4, (1 << 22) + 1, 150, 64) == 0
    assert lib.pkv_attention_workspace_bytes(ctypes.byref(d), 4, 0, 150, 64) == 0
    st = lib.pkv_paged_attention(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, (1 << 22) + 1, 150, 0.1,
                                 64, FAKE, None, 0, None)
    assert st == EUNSUPPORTED
    st = lib.pkv_paged_attention(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 16, FAKE, 4, 0, 150, 0.1,
                                 64, FAKE, None, 0, None)
    assert st == EINVAL
    # the prefill route needs no workspace: with zero sequences nothing is launched
    assert lib.pkv_paged_attention(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 16, FAKE, 0, 64, 150, 0.1,
                                   64, FAKE, None, 0, None) == 0


def test_shared_decode_sizing_and_checks():
    """Shared-prefix decode: with no prefix the workspace is the decode's; the
    prefix must be whole blocks, no longer than the length bound or the table
    (checked before anything is launched); zero sequences launch nothing."""
    lib = ops.library()
    d = _desc()                                 # block size 16
    assert lib.pkv_shared_decode_workspace_bytes(ctypes.byref(d), 4, 150, 0, 64) == \
        lib.pkv_decode_workspace_bytes(ctypes.byref(d), 4, 150, 64)
    assert lib.pkv_shared_decode_workspace_bytes(ctypes.byref(d), 4, 150, 24, 64) == 0   # not whole blocks
    assert lib.pkv_shared_decode_workspace_bytes(ctypes.byref(d), 4, 150, 160, 64) == 0  # past the bound
    args = lambda P, mctx, seqs=4, mb=16: (ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, mb, FAKE, seqs, mctx, P, 0.1,
                                          64, FAKE, FAKE, 1 << 30, None)
    assert lib.pkv_paged_decode_shared(*args(24, 150)) == EINVAL
    assert lib.pkv_paged_decode_shared(*args(160, 150)) == EINVAL
    assert lib.pkv_paged_decode_shared(*args(-16, 150)) == EINVAL
    assert lib.pkv_paged_decode_shared(*args(64, 150, mb=3)) == EINVAL                 # 4 blocks, table of 3
    assert lib.pkv_paged_decode_shared(*args(64, 150, seqs=0)) == 0


def test_shared_prefix_policy():
    """The cascade is chosen from 192 MiB of avoided prefix re-reads: with 8 kv
    heads, head_dim 128 and bf16 (4 KiB per token), a 2,000-token prefix pays
    from 26 sequences, a 4,096-token one from 13; fp8 needs about twice as many."""
    lib = ops.library()
    d = _desc(num_kv_heads=8, num_q_heads=32)
    pays = lambda B, P, dd=d: lib.pkv_shared_prefix_pays(ctypes.byref(dd), B, P)
    assert [pays(B, 2000) for B in (8, 16, 25, 26, 32, 256)] == [0, 0, 0, 1, 1, 1]
    assert [pays(B, 4096) for B in (8, 12, 13, 256)] == [0, 0, 1, 1]
    assert pays(1, 10 ** 6) == 0 and pays(256, 0) == 0
    fp8 = _desc(num_kv_heads=8, num_q_heads=32, kv_dtype=2, q_dtype=1, k_scale=FAKE, v_scale=FAKE)
    assert pays(26, 2000, fp8) == 0 and pays(50, 2000, fp8) == 0 and pays(51, 2000, fp8) == 1
    assert pays(-1, 16) == EINVAL


def test_strerror_and_version():
    lib = ops.library()
    assert lib.pkv_strerror(0) == b"ok"
    assert b"workspace" in lib.pkv_strerror(EWORKSPACE)
    assert lib.pkv_strerror(12345) == b"unknown status"
    assert b"gfx950" in lib.pkv_version()


def test_static_decode_checks_arguments_before_any_hip_call():
    """pkv_paged_decode_static: the decode's argument checks, on the host."""
    lib = ops.library()
    d = _desc()
    assert lib.pkv_paged_decode_static(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 64, 0.1,
                                       None, None) == EINVAL      # no output
    assert lib.pkv_paged_decode_static(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0, FAKE, 2, 64, 0.1,
                                       FAKE, None) == EINVAL      # no table columns
    assert lib.pkv_paged_decode_static(ctypes.byref(_desc(head_dim=96)), FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 64,
                                       0.1, FAKE, None) == EUNSUPPORTED
    assert lib.pkv_strerror(-6).decode().startswith("the decode needs more")


def test_probe_e4m3_calls_check_arguments():
    from paged_kv_cache_23_amd.build import PROBE_PATH

    lib = ctypes.CDLL(PROBE_PATH)
    P = ctypes.c_void_p
    chk, enc = lib.pkv_probe_e4m3_check, lib.pkv_probe_e4m3_encode
    chk.restype, chk.argtypes = ctypes.c_int, [ctypes.c_uint64, ctypes.c_uint64, P, P, P]
    enc.restype, enc.argtypes = ctypes.c_int, [P, P, ctypes.c_int64, P]
    assert chk(0, 16, None, FAKE, None) == -1
    assert chk(0, 0, FAKE, FAKE, None) == -1
    assert chk(1, 1 << 32, FAKE, FAKE, None) == -1          # past 2^32
    assert chk((1 << 32) - 4, 8, FAKE, FAKE, None) == -1
    assert enc(None, FAKE, 4, None) == -1 and enc(FAKE, FAKE, 0, None) == -1


def test_probe_library_exports_its_entry_point_and_checks_arguments():
    """libpkv_probe.so (the read-stream ceiling probe bench.py --tile-probe
    times) exports what include/pkv_probe.h declares and rejects bad
    arguments before any launch."""
    from paged_kv_cache_23_amd.build import PROBE_PATH

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "pkv_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))
    assert names == ["pkv_probe_e4m3_check", "pkv_probe_e4m3_encode", "pkv_probe_read_tiles"]
    lib = ctypes.CDLL(PROBE_PATH)
    fn = lib.pkv_probe_read_tiles
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    fn.restype, fn.argtypes = ctypes.c_int, [P, SZ, P, I64, I32, I32, I32, I32, P, P]
    ok = dict(buf=FAKE, nbytes=1 << 20, ids=FAKE, n=4, kib=4, inflight=16, waves=8, nt=1, sink=FAKE)
    for bad in (dict(buf=None), dict(kib=3), dict(kib=128), dict(inflight=12), dict(waves=6), dict(n=0),
                dict(nbytes=1024), dict(sink=None)):
        a = dict(ok, **bad)
        assert fn(a["buf"], a["nbytes"], a["ids"], a["n"], a["kib"], a["inflight"], a["waves"], a["nt"],
                  a["sink"], None) == -1, bad
