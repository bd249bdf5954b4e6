"""Pins for the oracle's FP8 sliding-window branch (CPU).

E4M3FN encoding: every code's own value encodes back to it; values from the
OCP format's definition worked by hand; brute-force nearest-code search with
exact rational arithmetic on random and tie values.  Row quantiser: the
row maximum lands on 448, the scale is amax/448, the error stays inside half
a code step, and scaling a row by a power of two scales only s.  Attention:
with no window it is the sparse attention; with no selection it is plain
softmax attention over the window (torch's scaled_dot_product_attention,
float64); the joint softmax equals the log-sum-exp merge of the two
branches (scipy's logsumexp); the window holds exactly the last W positions.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import workloads as W
from oracle import quantize as Q
from oracle import swa as S
from oracle.attend import sparse_attend
from oracle.formats import E4M3_TABLE
from oracle.step import Cache, FULL, REINDEX, REUSE, decode_step


def test_every_code_value_encodes_to_itself():
    for byte in list(range(0x00, 0x7F)) + list(range(0x80, 0xFF)):
        v = E4M3_TABLE[byte]
        assert int(S.e4m3_code(np.float64(v))) == byte, hex(byte)


@pytest.mark.parametrize("value,byte", [
    (1.0, 0x38), (-0.5, 0xB0), (3.0, 0x44), (448.0, 0x7E), (240.0, 0x77),
    (0.3, 0x2A),                       # between 0.28125 and 0.3125, above their midpoint
    (2.0 ** -10, 0x00),                # half the smallest subnormal: tie -> even code 0
    (3 * 2.0 ** -10, 0x02),            # tie between codes 1 and 2 -> 2
    (-(2.0 ** -11), 0x80),             # rounds to zero, sign kept
    (17.0, 0x58),                      # tie between 16 (0x58) and 18 (0x59) -> 16
    (19.0, 0x5A),                      # tie between 18 (0x59) and 20 (0x5A) -> 20
    (500.0, 0x7E), (-1e6, 0xFE),       # saturate at 448
])
def test_e4m3_worked_values(value, byte):
    assert int(S.e4m3_code(np.float64(value))) == byte


def _brute_code(y):
    """Nearest E4M3FN code by exhaustive search in exact rationals, ties to
    the even code, saturating; the sign bit is kept."""
    fy = Fraction(abs(float(y)))
    best, best_d = None, None
    for byte in range(0x00, 0x7F):
        d = abs(Fraction(float(E4M3_TABLE[byte])) - fy)
        if best is None or d < best_d or (d == best_d and byte % 2 == 0):
            best, best_d = byte, d
    return best | (0x80 if np.signbit(y) else 0)


def test_e4m3_matches_brute_force_nearest_search():
    rng = np.random.default_rng(5)
    ys = list((rng.standard_normal(300) * 2.0 ** rng.integers(-12, 9, 300)).astype(np.float32))
    mids = (E4M3_TABLE[:0x7E] + E4M3_TABLE[1:0x7F]) / 2
    ys += list(mids[rng.choice(mids.size, 60, replace=False)])            # exact ties
    ys += [np.nextafter(np.float32(m), np.float32(np.inf)) for m in mids[:40:3]]
    ys += [-v for v in ys[:50]] + [0.0, -0.0, 447.9, 448.5, 1e30]
    for y in ys:
        assert int(S.e4m3_code(np.float64(y))) == _brute_code(np.float64(y)), y


def test_row_quantiser_scale_maximum_and_error_bound():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((40, 512)) * 2.0 ** rng.integers(-8, 8, (40, 1))).astype(np.float32)
    codes, s = S.quantize_fp8_rows(x)
    amax = np.abs(x).max(axis=1)
    assert s.dtype == np.float32
    assert np.array_equal(s, (amax / np.float32(448.0)).astype(np.float32))
    top = np.argmax(np.abs(x), axis=1)
    assert np.all((codes[np.arange(40), top] & 0x7F) == 0x7E)
    v = S.dequantize_fp8_rows(codes, s)
    y = np.abs(x.astype(np.float64)) / s[:, None].astype(np.float64)
    bound = s[:, None] * (2.0 ** -4 * y * (1 + 2.0 ** -20) + 2.0 ** -10)
    assert np.all(np.abs(v - x) <= bound)
    assert np.all(np.signbit(v) == np.signbit(x))


def test_row_quantiser_worked_row_and_zero_rows():
    x = np.zeros((3, 512), dtype=np.float32)
    x[0, :8] = [448.0, 1.0, -0.5, 3.0, 0.3, 2.0 ** -10, 3 * 2.0 ** -10, 17.0]
    x[2, 5] = -0.0
    codes, s = S.quantize_fp8_rows(x)
    assert s[0] == 1.0 and s[1] == 0.0 and s[2] == 0.0
    assert list(codes[0, :8]) == [0x7E, 0x38, 0xB0, 0x44, 0x2A, 0x00, 0x02, 0x58]
    assert np.all(codes[0, 8:] == 0) and np.all(codes[1] == 0)
    assert codes[2, 5] == 0x80 and np.count_nonzero(codes[2]) == 1


def test_power_of_two_row_scaling_changes_only_the_scale():
    x = W.kv_rows(0, 0, 0, 0, 16)
    c0, s0 = S.quantize_fp8_rows(x)
    for k in (-5, 3):
        c1, s1 = S.quantize_fp8_rows((x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** k)).astype(np.float32))


def test_quantiser_rejects_non_finite():
    x = np.zeros((1, 512), dtype=np.float32)
    x[0, 3] = np.inf
    with pytest.raises(ValueError):
        S.quantize_fp8_rows(x)


def _setup(n, wlen, seed=1):
    c, s = Q.quantize_rows(W.kv_rows(0, seed, 0, 0, n))
    sc, ss = S.quantize_fp8_rows(W.kv_rows(0, seed + 50, 0, 0, wlen))
    return c, s, sc, ss


def test_no_window_is_the_sparse_attention():
    n = 8 * 20 + 3
    c, s, sc, ss = _setup(n, n)
    q = W.queries(0, 0, 0, 1, 16)[0]
    idx = np.int32([3, 0, 20, -1, 7])
    got = S.attend_with_window(c, s, n, q, idx, 0.05, sc, ss, n, 0)
    assert np.array_equal(got, sparse_attend(c, s, n, q, idx, 0.05))


def test_no_selection_is_plain_attention_over_the_window():
    n, win = 300, 77
    c, s, sc, ss = _setup(n, n)
    q = W.queries(0, 1, 0, 1, 16)[0]
    got = S.attend_with_window(c, s, n, q, np.full(4, -1, np.int32), 0.05, sc, ss, n, win)
    kv = torch.from_numpy(S.dequantize_fp8_rows(sc[n - win:], ss[n - win:]))
    qt = torch.from_numpy(q.astype(np.float64))
    want = torch.nn.functional.scaled_dot_product_attention(qt[None], kv[None], kv[None], scale=0.05)[0]
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-13)


def test_joint_softmax_is_the_log_sum_exp_merge_of_the_branches():
    n, win = 8 * 30, 100
    c, s, sc, ss = _setup(n, n)
    q = W.queries(0, 2, 0, 1, 8)[0].astype(np.float64)
    idx = np.int32([1, 4, 9, 29, 17])
    scale = 0.06
    got = S.attend_with_window(c, s, n, q, idx, scale, sc, ss, n, win)
    o1 = sparse_attend(c, s, n, q, idx, scale)
    o2 = S.attend_with_window(c, s, n, q, np.full(5, -1, np.int32), scale, sc, ss, n, win)
    from oracle.attend import gather_positions
    k1 = Q.dequantize_rows(c[gather_positions(idx, n)], s[gather_positions(idx, n)]).astype(np.float64)
    k2 = S.dequantize_fp8_rows(sc[n - win:], ss[n - win:])
    a1 = logsumexp(q @ k1.T * scale, axis=1)[:, None]
    a2 = logsumexp(q @ k2.T * scale, axis=1)[:, None]
    w1 = 1.0 / (1.0 + np.exp(a2 - a1))
    np.testing.assert_allclose(got, w1 * o1 + (1 - w1) * o2, rtol=1e-11, atol=1e-12)


def test_window_is_exactly_the_last_w_positions():
    n, win = 200, 64
    c, s, sc, ss = _setup(n, n)
    q = W.queries(0, 3, 0, 1, 16)[0]
    idx = np.int32([0, 5])
    base = S.attend_with_window(c, s, n, q, idx, 0.05, sc, ss, n, win)
    for p, changes in ((n - win - 1, False), (n - win, True), (n - 1, True)):
        ss2 = ss.copy()
        ss2[p] *= np.float32(2.0)
        got = S.attend_with_window(c, s, n, q, idx, 0.05, sc, ss2, n, win)
        assert (not np.array_equal(got, base)) == changes, p
    # a window wider than the sequence covers every position
    assert np.array_equal(S.window_positions(5, 64), np.arange(5))
    assert S.window_positions(0, 64).size == 0


def test_decode_step_local_branch_per_layer():
    B, H, K, n0, win = 2, 16, 4, 8 * 12 + 2, 40
    rng = np.random.default_rng(3)
    cache = Cache(B, 8 * 16)
    for b in range(B):
        cache.write(b, 0, W.kv_rows(0, 7, b, 0, n0))
        cache.seq_len[b] = n0
    swas = []
    for l in range(3):
        sw = S.SwaCache(B, 8 * 16)
        for b in range(B):
            sw.write(b, 0, W.kv_rows(0, 20 + l, b, 0, n0))
            sw.seq_len[b] = n0
        swas.append(sw)
    layers = [(FULL, 0, W.queries(0, l, 0, B, H)) for l in range(1)] + \
             [(REINDEX, 0, W.queries(0, 1, 0, B, H)), (REUSE, 0, W.queries(0, 2, 0, B, H))]
    new = rng.standard_normal((1, B, 512)).astype(np.float32)
    srows = rng.standard_normal((3, B, 512)).astype(np.float32)
    res = decode_step([cache], layers, new, K, 0, 0.05, swa=swas, swa_rows=srows, window=win)
    for l, sw in enumerate(swas):
        assert np.all(sw.seq_len == n0 + 1)
        for b in range(B):
            c8, s8 = S.quantize_fp8_rows(srows[l, b:b + 1])
            assert np.array_equal(sw.codes[b, n0], c8[0]) and sw.scales[b, n0] == s8[0]
            want = S.attend_with_window(cache.codes[b], cache.scales[b], n0 + 1, layers[l][2][b],
                                        res["idx"][l][b], 0.05, sw.codes[b], sw.scales[b], n0 + 1, win)
            assert np.array_equal(res["out"][l][b], want)
