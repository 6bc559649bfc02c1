"""The read-stream ceiling probe (libpkv_probe.so, bench.py --tile-probe)
reads exactly the tiles it is given: every lane's checksum equals the XOR,
computed here with NumPy, of the 16-byte pieces the probe's contract says
that lane reads.  So the ceiling it reports is the rate of that access
pattern and nothing less."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from paged_kv_cache_23_amd.build import PROBE_PATH

pytestmark = pytest.mark.gpu


def _lib():
    lib = ctypes.CDLL(PROBE_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.pkv_probe_read_tiles.restype = ctypes.c_int
    lib.pkv_probe_read_tiles.argtypes = [P, SZ, P, I64, I32, I32, I32, I32, P, P]
    return lib


def _expected(buf_u32: np.ndarray, ids: np.ndarray, tile_kib: int, waves: int) -> np.ndarray:
    """sink[w * 64 + lane] as the header defines it."""
    kib = buf_u32.reshape(-1, 64, 4)                          # [KiB][lane][4 words]
    buf_tiles = kib.shape[0] // tile_kib
    tiles = np.minimum(ids.astype(np.int64), buf_tiles - 1)
    pieces = tiles[:, None] * tile_kib + np.arange(tile_kib)[None, :]   # KiB index of each piece
    pieces = pieces.reshape(-1)
    per = -(-pieces.size // waves)
    out = np.zeros((waves, 64), dtype=np.uint32)
    for w in range(waves):
        p = pieces[w * per:(w + 1) * per]
        if p.size:
            x = np.bitwise_xor.reduce(kib[p], axis=0)                 # [64][4]
            out[w] = x[:, 0] ^ x[:, 1] ^ x[:, 2] ^ x[:, 3]
    return out.reshape(-1)


@pytest.mark.parametrize("tile_kib,inflight,nt", [(4, 16, 1), (2, 8, 0), (1, 32, 1), (8, 4, 0)])
def test_probe_reads_the_tiles_it_is_given(tile_kib, inflight, nt):
    rng = np.random.default_rng(tile_kib * 100 + inflight)
    nbytes = 8 << 20
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf_tiles = nbytes // (tile_kib << 10)
    ids = rng.permutation(buf_tiles).astype(np.uint32)[: buf_tiles - 3]
    ids[5] = buf_tiles + 7                                      # past the buffer: clamped to the last tile
    waves = 256
    dev = torch.device("cuda:0")
    buf = torch.from_numpy(host.view(np.int32)).to(dev)
    tid = torch.from_numpy(ids.view(np.int32)).to(dev)
    sink = torch.zeros(waves * 64, dtype=torch.int32, device=dev)
    lib = _lib()
    assert lib.pkv_probe_read_tiles(buf.data_ptr(), nbytes, tid.data_ptr(), ids.size, tile_kib, inflight, waves, nt,
                                    sink.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    got = sink.cpu().numpy().view(np.uint32)
    want = _expected(host, ids, tile_kib, waves)
    assert np.array_equal(got, want)
