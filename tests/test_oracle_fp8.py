"""Pins for the oracle's FP8 E4M3FN codec (CPU only).

Pinned against: the OCP OFP8 special values (tests/golden), torch's
float8_e4m3fn conversion (a library routine, valid for |x| < 464 where it does
not overflow to NaN), exhaustive round trips, and every rounding midpoint.
"""

import os

import numpy as np
import pytest
import torch

from oracle import fp8_decode, fp8_encode, fp8_finite_values

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_constants.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            rows.append((int(code, 16), float(val)))
    return rows


def test_ocp_special_values():
    for code, val in _golden():
        got = fp8_decode(np.array([code], np.uint8))[0]
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (hex(code), got, val)


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_value_table_shape():
    v = fp8_finite_values()
    assert len(v) == 127 and v[0] == 0.0 and v[-1] == 448.0
    assert np.all(np.diff(v) > 0)                      # strictly increasing
    assert np.count_nonzero(v < 2.0 ** -6) == 8        # zero + 7 subnormals


def test_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = fp8_decode(codes).astype(np.float32)
    assert np.array_equal(fp8_encode(vals), codes)


def _midpoints():
    v = fp8_finite_values()
    mids = (v[:-1] + v[1:]) / 2.0
    return mids.astype(np.float32)


def test_midpoints_tie_to_even_and_neighbours():
    mids = _midpoints()
    assert np.array_equal(mids.astype(np.float64), (fp8_finite_values()[:-1] + fp8_finite_values()[1:]) / 2)
    codes = fp8_encode(mids)
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(codes, expect.astype(np.uint8))
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    assert np.array_equal(fp8_encode(up), (lo + 1).astype(np.uint8))
    assert np.array_equal(fp8_encode(dn), lo.astype(np.uint8))
    assert np.array_equal(fp8_encode(-mids), (expect | 0x80).astype(np.uint8))


def test_matches_torch_below_464():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(30),
        rng.uniform(-463.9, 463.9, 200000).astype(np.float32),
        (rng.standard_normal(100000) * 1e-3).astype(np.float32),
        _midpoints(), -_midpoints(),
        np.nextafter(_midpoints(), np.float32(np.inf)),
        np.nextafter(_midpoints(), np.float32(0)),
        np.array([0.0, -0.0, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 463.99997], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8_encode(x), ref)


def test_saturation_and_nan():
    x = np.array([448, 464, 480, 1e30, np.inf, -464, -np.inf, np.nan], np.float32)
    assert list(fp8_encode(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F]


def test_planted_mistake_is_caught():
    """A codec that rounds ties away from zero must fail the midpoint pin."""
    v = fp8_finite_values()
    mids = _midpoints().astype(np.float64)
    away = np.searchsorted(v, mids, side="right")     # ties resolved upward
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert not np.array_equal(away, expect)
