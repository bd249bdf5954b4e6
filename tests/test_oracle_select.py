"""Pins for the oracle's top-k selection (CPU).

Pins: the defining property checked pair by pair (every kept block beats
every dropped one under (score desc, id asc)), nesting of top-k inside the
pool, padding, and the pages' pool size.
"""
import itertools

import numpy as np
import pytest

from oracle.select import select


def _check_defining_property(ids, scores, k, out):
    kept = [int(v) for v in out if v >= 0]
    assert kept == sorted(kept)
    assert len(kept) == min(k, len(ids))
    assert all(v == -1 for v in out[len(kept):])
    pos = {int(i): j for j, i in enumerate(ids)}
    dropped = [int(i) for i in ids if int(i) not in set(kept)]
    for a, b in itertools.product(kept, dropped):
        sa, sb = scores[pos[a]], scores[pos[b]]
        assert sa > sb or (sa == sb and a < b)


@pytest.mark.parametrize("seed", range(30))
def test_select_defining_property(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(1, 40))
    ids = rng.permutation(1000)[:m]
    scores = rng.integers(-3, 4, m).astype(np.float32)   # many ties
    k = int(rng.integers(1, 50))
    out = select(ids, scores, k)
    _check_defining_property(ids, scores, k, out)


def test_ties_go_to_lowest_id():
    ids = np.arange(10)
    out = select(ids, np.zeros(10, dtype=np.float32), 3)
    assert out.tolist() == [0, 1, 2]
    sc = np.float32([1, 5, 5, 5, 0, 5, 2, 2, 9, 5])
    assert select(ids, sc, 4).tolist() == [1, 2, 3, 8]


def test_signed_zero_is_a_tie():
    out = select([4, 2], np.float32([0.0, -0.0]), 1)
    # the pinned scores never hold -0; as floats -0 == +0, so the lower id wins
    assert out.tolist() == [2]


def test_nesting_and_pool_equals_flat():
    rng = np.random.default_rng(5)
    ids = np.arange(5000)
    scores = rng.standard_normal(5000).astype(np.float32)
    scores[rng.integers(0, 5000, 500)] = 0.25       # ties
    pool = select(ids, scores, 2048)
    top = select(ids, scores, 256)
    top_in_pool = select(pool, scores[pool], 256)
    assert np.array_equal(top, top_in_pool)
    assert set(top.tolist()) <= set(pool.tolist())
    assert np.array_equal(select(ids, scores, 5000), ids.astype(np.int32))


def test_fewer_candidates_than_k():
    out = select([7, 3], np.float32([1, 2]), 5)
    assert out.tolist() == [3, 7, -1, -1, -1]
    assert select([], np.float32([]), 3).tolist() == [-1, -1, -1]


def test_pool_size_from_pages(golden):
    assert golden["pool_blocks"] * golden["block_positions"] == golden["pool_positions"]
