"""Pins for the oracle's per-head indexer variant (score = best per-head
score, each head scored in the pinned float32 order) (CPU).

Pins: one head reduces to the collapsed score of that head; hand-worked
inputs whose every float32 step is exact equal the exact rational maximum
over heads (Fractions); on random inputs the result lies within the
dot-product error bound of the exact maximum; the result is invariant under
a permutation of the heads and is one of the heads' own scores; a case where
summing the heads and taking the best head pick different blocks; the
decode-step driver threads the rule through every selecting layer.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import indexer as I
from oracle import quantize as Q
from oracle.select import select
from oracle.step import FULL, REINDEX, REUSE, Cache, decode_step


def _keys(n, seed_cache=0):
    c, s = Q.quantize_rows(W.kv_rows(0, seed_cache, 0, 0, n))
    return c, s, I.block_keys(c, s, n)


def _exact_dot(q, k):
    return sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q, k))


def test_one_head_is_that_heads_pinned_score():
    _, _, keys = _keys(8 * 40 + 3)
    q = W.queries(0, 3, 0, 1, 1)[0]
    assert np.array_equal(I.headmax_scores_from_keys(q, keys).view(np.uint32),
                          I.block_scores_from_keys(q[0], keys).view(np.uint32))


def test_hand_worked_exact_maximum():
    # keys in half-integers, queries small integers: every product and every
    # partial sum is a multiple of 1/2 below 2^24, so each float32 step is
    # exact and the result must equal the exact rational maximum over heads
    rng = np.random.default_rng(11)
    keys = (rng.integers(-4, 5, (6, 512)) / 2).astype(np.float32)
    q = rng.integers(-3, 4, (5, 512)).astype(np.float32)
    got = I.headmax_scores_from_keys(q, keys)
    for b in range(6):
        exact = max(_exact_dot(q[h], keys[b]) for h in range(5))
        assert Fraction(float(got[b])) == exact
    # the same keys, one head doubled: its score doubles exactly and wins
    q2 = q.copy()
    best = int(np.argmax([float(_exact_dot(q[h], keys[0])) for h in range(5)]))
    q2[best] *= 2
    assert Fraction(float(I.headmax_scores_from_keys(q2, keys)[0])) == 2 * _exact_dot(q[best], keys[0])


def _gamma(n):
    u = Fraction(1, 2 ** 24)
    return n * u / (1 - n * u)


def test_within_error_bound_of_exact_maximum():
    _, _, keys = _keys(8 * 24, seed_cache=1)
    q = W.queries(0, 4, 0, 1, 8)[0]
    got = I.headmax_scores_from_keys(q, keys)
    g = _gamma(1 + 15 + 5)
    for b in range(0, 24, 5):
        exact = [_exact_dot(q[h], keys[b]) for h in range(8)]
        bound = max(g * sum(abs(Fraction(float(a)) * Fraction(float(k))) for a, k in zip(q[h], keys[b]))
                    for h in range(8))
        assert abs(Fraction(float(got[b])) - max(exact)) <= bound


def test_permutation_invariant_and_attained():
    _, _, keys = _keys(8 * 33 + 1, seed_cache=2)
    q = W.queries(0, 5, 0, 1, 16)[0]
    got = I.headmax_scores_from_keys(q, keys)
    perm = np.random.default_rng(5).permutation(16)
    assert np.array_equal(got.view(np.uint32), I.headmax_scores_from_keys(q[perm], keys).view(np.uint32))
    per_head = np.stack([I.block_scores_from_keys(q[h], keys) for h in range(16)])
    assert np.all(got >= per_head)
    assert np.all(np.any(per_head == got[None, :], axis=0))


def test_sum_and_max_pick_different_blocks():
    # head A: block 0 -> 3, block 1 -> -10; head B: block 0 -> -1, block 1 -> 4.
    # Summing the heads prefers block 0 (2 > -6); the best head prefers block 1 (4 > 3).
    keys = np.zeros((2, 512), dtype=np.float32)
    keys[0, 0], keys[0, 16] = 3.0, -1.0
    keys[1, 0], keys[1, 16] = -10.0, 4.0
    q = np.zeros((2, 512), dtype=np.float32)
    q[0, 0] = 1.0                       # head A reads channel 0
    q[1, 16] = 1.0                      # head B reads channel 16
    ids = np.arange(2)
    summed = I.block_scores_from_keys(I.collapse_query(q), keys)
    best = I.headmax_scores_from_keys(q, keys)
    assert summed.tolist() == [2.0, -6.0] and best.tolist() == [3.0, 4.0]
    assert select(ids, summed, 1).tolist() == [0]
    assert select(ids, best, 1).tolist() == [1]


def test_block_scores_rule_switch():
    n = 8 * 20 + 6
    c, s, keys = _keys(n, seed_cache=3)
    q = W.queries(0, 6, 0, 1, 16)[0]
    ids, sc = I.block_scores(c, s, n, q, cand=[4, 19, 0], score=I.SCORE_HEADMAX)
    assert ids.tolist() == [4, 19, 0]
    assert np.array_equal(sc, I.headmax_scores_from_keys(q, keys[[4, 19, 0]]))
    with pytest.raises(ValueError):
        I.block_scores(c, s, n, q, score=7)
    bad = q.copy()
    bad[3, 9] = np.inf
    with pytest.raises(ValueError):
        I.block_scores(c, s, n, bad, score=I.SCORE_HEADMAX)


def test_driver_uses_the_rule_in_every_selecting_layer():
    n, H, K, P = 1000, 16, 8, 32
    caches = []
    for ci in range(2):
        oc = Cache(2, 1008)
        for b in range(2):
            oc.write(b, 0, W.kv_rows(1, ci, b, 0, n))
            oc.seq_len[b] = n
        caches.append(oc)
    qs = [W.queries(1, l, 0, 2, H) for l in range(4)]
    layers = [(FULL, 0, qs[0]), (REINDEX, 0, qs[1]), (REUSE, 0, qs[2]), (FULL, 1, qs[3])]
    res = decode_step(caches, layers, None, K, P, 1 / np.sqrt(512), score=I.SCORE_HEADMAX)
    for b in range(2):
        ids, sc = I.block_scores(caches[0].codes[b], caches[0].scales[b], n, qs[0][b], score=I.SCORE_HEADMAX)
        assert np.array_equal(res["pool"][b], select(ids, sc, P))
        assert np.array_equal(res["idx"][0][b], select(ids, sc, K))          # nested in the pool
        ids1, sc1 = I.block_scores(caches[0].codes[b], caches[0].scales[b], n, qs[1][b], cand=res["pool"][b],
                                   score=I.SCORE_HEADMAX)
        assert np.array_equal(res["idx"][1][b], select(ids1, sc1, K))
        assert np.array_equal(res["idx"][2][b], res["idx"][1][b])
        ids3, sc3 = I.block_scores(caches[1].codes[b], caches[1].scales[b], n, qs[3][b], cand=res["pool"][b],
                                   score=I.SCORE_HEADMAX)
        assert np.array_equal(res["idx"][3][b], select(ids3, sc3, K))
