"""Pins for the oracle's row quantiser (CPU).

Pins: exact round trip of representable groups, the per-group error bound
max(s, amax - 6s), a brute-force nearest search with Fractions, the pages'
range argument on the synthetic rows, the byte budget, nibble order and the
sign of zero.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import quantize as Q


def _random_representable(rng, R):
    """Rows whose every group holds a +-6 code, so quantise(deq) is exact."""
    sb = rng.integers(1, 0x7F, (R, Q.NGROUPS)).astype(np.uint8)
    nib = rng.integers(0, 16, (R, Q.D)).astype(np.uint8)
    g = nib.reshape(R, Q.NGROUPS, Q.GROUP)
    pos = rng.integers(0, Q.GROUP, (R, Q.NGROUPS))
    sgn = rng.integers(0, 2, (R, Q.NGROUPS)).astype(np.uint8) << 3
    np.put_along_axis(g, pos[..., None], (sgn | 7)[..., None], axis=2)
    nib = g.reshape(R, Q.D)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes, sb


def test_round_trip_exact_on_representable_groups():
    rng = np.random.default_rng(10)
    codes, scales = _random_representable(rng, 300)
    x = Q.dequantize_rows(codes, scales)
    c2, s2 = Q.quantize_rows(x)
    assert np.array_equal(s2, scales)
    assert np.array_equal(c2, codes)


def test_error_bound_per_group():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((500, Q.D)) * np.exp2(rng.uniform(-12, 8, (500, 1)))).astype(np.float32)
    c, s = Q.quantize_rows(x)
    y = Q.dequantize_rows(c, s).astype(np.float64)
    err = np.abs(y - x).reshape(500, Q.NGROUPS, Q.GROUP).max(axis=2)
    amax = np.abs(x.astype(np.float64)).reshape(500, Q.NGROUPS, Q.GROUP).max(axis=2)
    sv = F.E4M3_TABLE[s]
    assert np.all(err <= np.maximum(sv, amax - 6 * sv))


def _nearest_even(value, grid):
    best = None
    for i, g in enumerate(grid):
        key = (abs(Fraction(g) - value), i % 2)
        if best is None or key < best[0]:
            best = (key, i)
    return best[1]


def test_brute_force_tiny_rows():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((3, Q.D)) * np.float32([[0.01], [1.0], [300.0]])).astype(np.float32)
    x[0, :16] = 0.0
    x[0, 3] = -0.0
    c, s = Q.quantize_rows(x)
    e4 = [F.e4m3_value(b) for b in range(0x7F)]
    nib = Q.unpack_codes(c)
    for r in range(3):
        for g in range(Q.NGROUPS):
            grp = x[r, 16 * g:16 * g + 16]
            amax = max(abs(Fraction(float(v))) for v in grp)
            sb = _nearest_even(amax / 6, e4)
            assert s[r, g] == sb
            sv = Fraction(e4[sb])
            for i, v in enumerate(grp.tolist()):
                mag = 0 if sv == 0 else _nearest_even(abs(Fraction(v)) / sv, F.E2M1_MAGNITUDES)
                want = (8 if np.signbit(np.float32(v)) else 0) | mag
                assert nib[r, 16 * g + i] == want


def test_sign_of_zero_and_nibble_order():
    x = np.zeros((1, Q.D), dtype=np.float32)
    x[0, 0] = -0.0
    x[0, 3] = 6.0        # group 0 scale 1.0; channel 3 -> code 7 in the high nibble of byte 1
    x[0, 2] = -0.5       # code 0x9 in the low nibble of byte 1
    c, s = Q.quantize_rows(x)
    assert F.e4m3_value(int(s[0, 0])) == 1.0
    assert c[0, 0] == 0x08          # ch0 = -0 -> 0x8, ch1 = +0 -> 0x0
    assert c[0, 1] == (0x7 << 4) | 0x9
    assert np.all(s[0, 1:] == 0)


def test_non_finite_rejected():
    x = np.zeros((1, Q.D), dtype=np.float32)
    x[0, 5] = np.nan
    with pytest.raises(ValueError):
        Q.quantize_rows(x)


def test_byte_budget(golden):
    assert Q.CODE_BYTES + Q.SCALE_BYTES == Q.BYTES_PER_TOKEN == 288
    assert Q.D == golden["latent_channels"]
    assert Q.GROUP == golden["channels_per_scale"]
    # 4-bit codes vs 16-bit storage: a quarter of the bytes
    assert 1 - (Q.CODE_BYTES / (Q.D * 2)) == golden["fp4_saving_vs_16bit"]


def test_range_argument_on_synthetic_rows(golden):
    rows = W.kv_rows(0, 0, 0, 0, 8192)
    norms = np.linalg.norm(rows.astype(np.float64), axis=1)
    bound = np.sqrt(512.0)
    assert abs(bound - golden["l2_bound"]) < 0.05
    assert np.all(norms <= bound * (1 + 1e-5))
    assert np.abs(rows).max() <= bound < golden["representable_max"]
    c, s = Q.quantize_rows(rows)
    deq = Q.dequantize_rows(c, s)
    assert np.abs(deq).max() <= golden["representable_max"]
    # the scales stay far from saturation on this data
    assert s.max() < 0x7E
