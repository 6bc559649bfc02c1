"""The float32 -> OCP E4M3FN conversion that the append kernels use for an
fp8 cache (Habr KV-Cache article, section 2: an fp8 cache stores one byte
per element; the rounding is this library's reading of the format:
nearest, ties to even, +-448 saturation, NaN kept).

The kernels convert with gfx950's v_cvt_pk_fp8_f32 on values clamped to
+-448 and put NaN codes back afterwards.  libpkv_probe.so runs that same
device function (csrc/e4m3.h) on every binary32 bit pattern, in both halves
of the two-value conversion, against the format's rounding written out on
the binary32 fields; and on a sample of inputs its codes are compared here
with the CPU oracle's encoder."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_23_amd.build import PROBE_PATH

pytestmark = pytest.mark.gpu


def _probe():
    lib = ctypes.CDLL(PROBE_PATH)
    P = ctypes.c_void_p
    lib.pkv_probe_e4m3_check.restype = ctypes.c_int
    lib.pkv_probe_e4m3_check.argtypes = [ctypes.c_uint64, ctypes.c_uint64, P, P, P]
    lib.pkv_probe_e4m3_encode.restype = ctypes.c_int
    lib.pkv_probe_e4m3_encode.argtypes = [P, P, ctypes.c_int64, P]
    return lib


def test_every_binary32_input_rounds_as_the_format_says():
    lib = _probe()
    dev = torch.device("cuda:0")
    bad = torch.zeros(1, dtype=torch.int64, device=dev)
    first_bad = torch.full((1,), -1, dtype=torch.int32, device=dev)   # 0xFFFFFFFF
    stream = torch.cuda.current_stream().cuda_stream
    print("E4M3 conversion: all 2^32 binary32 inputs", flush=True)
    for part in range(4):   # 2^30 inputs per launch
        assert lib.pkv_probe_e4m3_check(part << 30, 1 << 30, bad.data_ptr(), first_bad.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    n_bad = int(bad.item())
    assert n_bad == 0, f"{n_bad} inputs convert differently; the first is {int(first_bad.item()) & 0xFFFFFFFF:#010x}"


def test_codes_equal_the_oracles_encoder():
    rng = np.random.default_rng(12)
    bits = [rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)]
    # every pattern within 2^12 of the format's landmarks: 448 and the
    # saturation edge, 2^-6 (smallest normal), 2^-9 (smallest subnormal),
    # 2^-10 (half of it), 1, the infinities and the NaNs
    for base in (0x43E00000, 0x43E80000, 0x3C800000, 0x3B000000, 0x3A800000, 0x3F800000, 0x7F800000, 0x00000000):
        bits.append(((base + np.arange(-4096, 4096)) & 0xFFFFFFFF).astype(np.uint32))
    x = np.concatenate(bits)
    x = np.concatenate([x, x | np.uint32(0x80000000)]).view(np.float32)
    lib = _probe()
    dev = torch.device("cuda:0")
    xin = torch.from_numpy(x.copy()).to(dev)
    out = torch.empty(x.shape[0], dtype=torch.uint8, device=dev)
    assert lib.pkv_probe_e4m3_encode(xin.data_ptr(), out.data_ptr(), x.shape[0],
                                     torch.cuda.current_stream().cuda_stream) == 0
    got = out.cpu().numpy()
    with np.errstate(invalid="ignore"):
        want = oracle.e4m3_encode(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} codes differ, e.g. input {x.view(np.uint32)[bad[0]]:#010x}: " \
                          f"{got[bad[0]]:#04x} vs {want[bad[0]]:#04x}"
