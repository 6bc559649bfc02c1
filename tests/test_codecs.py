"""Pins of the oracle's number-format code: bf16 widening and OCP E4M3FN."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, e4m3_decode, e4m3_encode


def _all_bf16_bits():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_bf16_widening_matches_torch_on_every_pattern():
    bits = _all_bf16_bits()
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = bf16_bits_to_f64(bits)
    assert np.array_equal(got, ref, equal_nan=True)


def test_e4m3_decode_matches_torch_float8_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    assert np.array_equal(got, ref, equal_nan=True)
    # the format's landmarks: largest finite, smallest subnormal, NaN codes
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.count_nonzero(np.isnan(got)) == 2


def test_e4m3_decode_then_encode_is_identity_on_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), codes)


def _nearest_code_brute_force(x: float) -> int:
    """Nearest finite E4M3 value by exhaustive search; ties go to the even code;
    beyond 448 saturate; NaN keeps the sign bit."""
    if np.isnan(x):
        return 0x7F | (0x80 if np.signbit(x) else 0)
    table = e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # non-negative finite values, codes 0..126
    a = min(abs(float(x)), 1e300)
    if a >= 448.0:
        code = 0x7E
    else:
        d = np.abs(table - a)
        best = np.flatnonzero(d == d.min())
        code = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
    return code | (0x80 if np.signbit(x) else 0)


def test_e4m3_encode_matches_brute_force_on_every_bf16_value():
    vals = bf16_bits_to_f64(_all_bf16_bits()).astype(np.float32)
    got = e4m3_encode(vals)
    ref = np.array([_nearest_code_brute_force(v) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_matches_torch_cast_inside_the_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)]).astype(np.float32)
    x = x[np.abs(x) < 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3_encode(x), ref)


@pytest.mark.parametrize("x,code", [
    (0.0, 0x00), (-0.0, 0x80),
    (448.0, 0x7E), (-448.0, 0xFE),
    (464.0, 0x7E), (1e6, 0x7E), (float("inf"), 0x7E), (float("-inf"), 0xFE),
    (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),   # ties to even at the bottom
    (2.0 ** -6, 0x08), (1.0, 0x38), (1.0625, 0x38), (1.1875, 0x3A),   # 1 + 1/16 ties down, 1 + 3/16 ties up
    (240.0, 0x77), (248.0, 0x78), (15.5 * 2.0 ** -4, 0x38),
])
def test_e4m3_boundary_table(x, code):
    """Hand table from the E4M3FN definition: saturation, subnormals, ties."""
    assert int(e4m3_encode(np.float32(x))) == code
