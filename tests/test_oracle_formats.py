"""Pins for the oracle's number formats (CPU).

What pins them: the pages' constants (16 levels, 448, 6, 2688), the OCP
bit-field definitions written independently of the oracle's tables, torch's
float8_e4m3fn decode and round-to-nearest-even cast (a library routine), and
a brute-force exact nearest search with Fractions.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


def _e2m1_bitfield(n):
    # OCP MX E2M1: s | e(2) | m(1), bias 1; e == 0 is subnormal m * 2^-1
    s = -1 if n & 8 else 1
    e = (n >> 1) & 3
    m = n & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return s * mag


def test_e2m1_table_matches_bitfield_definition():
    for n in range(16):
        assert F.e2m1_value(n) == _e2m1_bitfield(n)


def test_e2m1_levels_and_max(golden):
    assert len(F.E2M1_TABLE) == golden["levels_4bit"] == 2 ** 4
    assert F.E2M1_MAX == golden["e2m1_max"] == np.max(F.E2M1_TABLE)
    # 16 codes, 15 distinct values (+0 and -0)
    assert len(set(F.E2M1_TABLE.tolist())) == 15


def test_e4m3_table_matches_torch_decode():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.E4M3_TABLE
    nan_t, nan_o = np.isnan(t), np.isnan(ours)
    assert np.array_equal(nan_t, nan_o)
    assert set(np.flatnonzero(nan_o).tolist()) == set(F.E4M3_NAN_BYTES)
    assert np.array_equal(t[~nan_t], ours[~nan_o])


def test_e4m3_max_and_range_product(golden):
    assert F.E4M3_MAX == golden["e4m3_max"] == np.nanmax(F.E4M3_TABLE)
    assert F.E4M3_MAX * F.E2M1_MAX == golden["representable_max"]
    assert F.e4m3_value(0x01) == 2.0 ** -9     # smallest subnormal
    assert F.e4m3_value(0x08) == 2.0 ** -6     # smallest normal
    assert F.e4m3_value(0x38) == 1.0


def test_e4m3_encoder_matches_torch_rne_cast():
    rng = np.random.default_rng(1)
    # y with few significant bits so 6*y is exact in float32; y in [0, 464]
    y = np.concatenate([
        rng.uniform(0, 464, 20000),
        np.exp2(rng.uniform(-12, 9, 20000)),
    ]).astype(np.float32)
    y = (np.round(y * 2.0 ** 12) / 2.0 ** 12).astype(np.float32)
    y = y[(y <= 464) & (y * 6 == (y.astype(np.float64) * 6))]
    mids = (F.E4M3_MIDPOINTS[:126]).astype(np.float32)   # all ties too
    y = np.concatenate([y, mids, np.float32([0, 448, 464, 2.0 ** -10])])
    ours = F.e4m3_scale_byte(y.astype(np.float64) * 6)
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def _nearest_even(value: Fraction, grid):
    """Brute force: the grid index nearest to value, ties to the even index;
    beyond the grid saturates."""
    best = None
    for i, g in enumerate(grid):
        d = abs(Fraction(g) - value)
        key = (d, i % 2)
        if best is None or key < best[0]:
            best = (key, i)
    return best[1]


def test_e4m3_encoder_brute_force():
    grid = [F.e4m3_value(b) for b in range(0x7F)]
    rng = np.random.default_rng(2)
    amax = np.concatenate([
        np.exp2(rng.uniform(-14, 12, 3000)).astype(np.float32),
        (6 * F.E4M3_MIDPOINTS).astype(np.float32)[::5],
        np.float32([0, 6 * 448, 6 * 460, 1e6]),
    ])
    ours = F.e4m3_scale_byte(amax.astype(np.float64))
    for a, o in zip(amax.tolist(), ours.tolist()):
        assert o == _nearest_even(Fraction(a) / 6, grid), a


def test_e2m1_tie_table():
    # |x|/s at each midpoint rounds to the even code
    s = 1.0
    cases = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
             6.0: 6.0, 7.0: 6.0, 100.0: 6.0, 0.2499: 0.0, 0.2501: 0.5}
    for v, want in cases.items():
        code = int(F.e2m1_magnitude_code(np.float64(v), np.float64(s)))
        assert F.E2M1_MAGNITUDES[code] == want, v


def test_e2m1_encoder_brute_force():
    rng = np.random.default_rng(3)
    grid = list(F.E2M1_MAGNITUDES)
    svals = [F.e4m3_value(b) for b in rng.integers(1, 0x7F, 200)]
    for s in svals:
        x = (np.abs(rng.standard_normal(40)) * s * rng.uniform(0.5, 8)).astype(np.float32)
        x = np.concatenate([x, (np.float64(s) * F.E2M1_MIDPOINTS).astype(np.float32)])
        codes = F.e2m1_magnitude_code(x.astype(np.float64), np.float64(s))
        for xi, c in zip(x.tolist(), codes.tolist()):
            assert c == _nearest_even(Fraction(xi) / Fraction(s), grid), (xi, s)
    # zero scale: magnitude 0
    assert int(F.e2m1_magnitude_code(np.float64(0.001), np.float64(0.0))) == 0
