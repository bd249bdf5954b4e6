"""Pins for the oracle's indexer: block keys, query collapse, pinned scores (CPU).

Pins: block sums equal the exact rational sums (Fractions), keys are the
exact mean for full blocks; scores lie within the recursive dot-product
error bound of the exact value; a unit query picks one key channel exactly;
hand-worked float32 cases fix the summation order; the literal scalar loop
and the array form agree bit for bit.
"""
from fractions import Fraction

import numpy as np

import workloads as W
from oracle import indexer as I
from oracle import quantize as Q


def _cache(n, wid=0, seed_cache=0):
    rows = W.kv_rows(wid, seed_cache, 0, 0, n)
    return Q.quantize_rows(rows)


def test_block_sums_exact_and_key_is_mean():
    n = 8 * 40 + 5
    c, s = _cache(n)
    keys = I.block_keys(c, s, n)
    deq = Q.dequantize_rows(c, s)
    assert keys.shape == (41, 512)
    for b in range(41):
        cnt = min(8, n - 8 * b)
        for ch in range(0, 512, 37):
            exact = sum(Fraction(float(deq[8 * b + t, ch])) for t in range(cnt))
            if cnt == 8:
                assert Fraction(float(keys[b, ch])) == exact / 8
            else:
                # the float32 sum is exact here, then one float32 division
                assert keys[b, ch] == np.float32(float(exact)) / np.float32(cnt)
                assert abs(Fraction(float(keys[b, ch])) - exact / cnt) <= abs(exact / cnt) * Fraction(1, 2 ** 24)


def test_collapse_query_order_and_exactness():
    q = np.zeros((64, 512), dtype=np.float32)
    q[0] = 1.0
    q[1:] = 2.0 ** -24          # each add ties and rounds back to 1.0
    assert np.all(I.collapse_query(q) == 1.0)
    rng = np.random.default_rng(4)
    qi = rng.integers(-1000, 1000, (16, 512)).astype(np.float32)
    assert np.array_equal(I.collapse_query(qi), qi.astype(np.int64).sum(0).astype(np.float32))


def _gamma(n):
    u = Fraction(1, 2 ** 24)
    return n * u / (1 - n * u)


def test_score_within_dot_product_error_bound():
    n = 8 * 64
    c, s = _cache(n, seed_cache=1)
    keys = I.block_keys(c, s, n)
    q = W.queries(0, 0, 0, 1, 16)[0]
    qbar = I.collapse_query(q)
    scores = I.block_scores_from_keys(qbar, keys)
    g = _gamma(1 + 15 + 5)
    for b in range(0, 64, 3):
        terms = [Fraction(float(qbar[ch])) * Fraction(float(keys[b, ch])) for ch in range(512)]
        exact = sum(terms)
        bound = g * sum(abs(t) for t in terms)
        assert abs(Fraction(float(scores[b])) - exact) <= bound


def test_unit_query_selects_one_channel():
    n = 8 * 16
    c, s = _cache(n)
    keys = I.block_keys(c, s, n)
    for ch in (0, 1, 15, 16, 255, 511):
        qbar = np.zeros(512, dtype=np.float32)
        qbar[ch] = 1.0
        sc = I.block_scores_from_keys(qbar, keys)
        assert np.array_equal(sc, keys[:, ch] + np.float32(0.0))
        qbar[ch] = -2.0
        sc = I.block_scores_from_keys(qbar, keys)
        assert np.array_equal(sc, -2 * keys[:, ch] + np.float32(0.0))


def test_summation_order_hand_worked():
    # within a group: left to right, so fifteen 2^-24 terms vanish against 1.0
    qbar = np.ones(512, dtype=np.float32)
    key = np.zeros(512, dtype=np.float32)
    key[0] = 1.0
    key[1:16] = 2.0 ** -24
    assert I.pinned_dot(qbar, key) == np.float32(1.0)
    # across groups: adjacent-pair tree; g0 = 1, g1..g31 = 2^-24 gives 1 + 15*2^-23
    key = np.zeros(512, dtype=np.float32)
    key[0] = 1.0
    key[16::16] = 2.0 ** -24
    assert I.pinned_dot(qbar, key) == np.float32(1.0 + 15 * 2.0 ** -23)
    # the sum of everything that cancels is +0, never -0
    key = np.zeros(512, dtype=np.float32)
    key[0], key[16] = -1.0, 1.0
    r = I.pinned_dot(qbar, key)
    assert r == 0 and not np.signbit(r)
    r = I.pinned_dot(-qbar, np.zeros(512, dtype=np.float32))
    assert r == 0 and not np.signbit(r)


def test_scalar_and_array_forms_agree():
    n = 8 * 50 + 7
    c, s = _cache(n, seed_cache=2)
    keys = I.block_keys(c, s, n)
    qbar = I.collapse_query(W.queries(0, 1, 0, 1, 64)[0])
    arr = I.block_scores_from_keys(qbar, keys)
    for b in range(keys.shape[0]):
        assert arr[b].tobytes() == I.pinned_dot(qbar, keys[b]).tobytes()


def test_block_scores_candidates():
    n = 8 * 30
    c, s = _cache(n)
    q = W.queries(0, 2, 0, 1, 16)[0]
    ids, sc = I.block_scores(c, s, n, q)
    ids2, sc2 = I.block_scores(c, s, n, q, cand=[29, 3, -1, 7])
    assert ids2.tolist() == [29, 3, 7]
    assert np.array_equal(sc2, sc[[29, 3, 7]])
