"""Pins for the oracle's layer-stack driver (CPU).

Pins: Reuse layers reproduce the earlier selection exactly; the first Full
layer's top-k equals the flat top-k of all blocks and lies in its pool; a
pool at least as large as the block count gives the flat result; Reindex
reads the latest Full cache; appends land at seq_len; malformed stacks fail.
"""
import numpy as np
import pytest

import workloads as W
from oracle import indexer as I
from oracle.select import select
from oracle.step import FULL, REINDEX, REUSE, Cache, decode_step


def _caches(n_caches, batch, n, cap=None):
    caches = []
    for ci in range(n_caches):
        cache = Cache(batch, cap or ((n + 16 + 7) // 8 * 8))
        for b in range(batch):
            cache.write(b, 0, W.kv_rows(0, ci, b, 0, n))
            cache.seq_len[b] = n
        caches.append(cache)
    return caches


def _layers(pattern, batch, heads, step=0):
    out, cur = [], -1
    for li, m in enumerate(pattern):
        if m == FULL:
            cur += 1
        out.append((m, cur, W.queries(0, li, step, batch, heads)))
    return out


def test_reuse_reproduces_previous_selection():
    pattern = (FULL, REINDEX, REUSE, REUSE, REINDEX)
    caches = _caches(1, 2, 8 * 100 + 3)
    r = decode_step(caches, _layers(pattern, 2, 4), None, topk=16, pool=40, scale=0.05)
    assert np.array_equal(r["idx"][2], r["idx"][1])
    assert np.array_equal(r["idx"][3], r["idx"][1])
    assert not np.array_equal(r["idx"][4], r["idx"][1])


def test_first_full_layer_nesting_and_flat_equivalence():
    caches = _caches(1, 1, 8 * 300)
    layers = _layers((FULL,), 1, 8)
    r = decode_step(caches, layers, None, topk=20, pool=64, scale=0.05)
    ids, sc = I.block_scores(caches[0].codes[0], caches[0].scales[0], 2400, layers[0][2][0])
    assert np.array_equal(r["idx"][0][0], select(ids, sc, 20))
    assert np.array_equal(r["pool"][0], select(ids, sc, 64))
    assert set(r["idx"][0][0].tolist()) <= set(r["pool"][0].tolist())


def test_pool_covering_all_blocks_equals_flat():
    pattern = (FULL, REINDEX, REINDEX)
    caches = _caches(1, 2, 8 * 50 + 1)
    layers = _layers(pattern, 2, 4)
    hier = decode_step(caches, layers, None, topk=8, pool=64, scale=0.05)
    flat = decode_step(caches, layers, None, topk=8, pool=0, scale=0.05)
    for a, b in zip(hier["idx"], flat["idx"]):
        assert np.array_equal(a, b)
    for a, b in zip(hier["out"], flat["out"]):
        assert np.array_equal(a, b)
    # 51 blocks padded to a 64-entry pool
    assert hier["pool"][0].tolist()[:51] == list(range(51))
    assert hier["pool"][0].tolist()[51:] == [-1] * 13


def test_reindex_reads_latest_full_cache_and_later_full_own_cache():
    pattern = (FULL, REINDEX, FULL, REINDEX)
    caches = _caches(2, 1, 8 * 60)
    layers = _layers(pattern, 1, 4)
    r = decode_step(caches, layers, None, topk=6, pool=0, scale=0.05)
    for li, ci in ((1, 0), (2, 1), (3, 1)):
        ids, sc = I.block_scores(caches[ci].codes[0], caches[ci].scales[0], 480, layers[li][2][0])
        assert np.array_equal(r["idx"][li][0], select(ids, sc, 6))


def test_append_then_layers():
    caches = _caches(1, 2, 13, cap=32)
    rows = W.append_rows(0, 0, 0, 2)[None]
    r = decode_step(caches, _layers((FULL,), 2, 2), rows, topk=4, pool=0, scale=0.05)
    assert caches[0].seq_len.tolist() == [14, 14]
    from oracle.quantize import quantize_rows
    c, s = quantize_rows(rows[0])
    assert np.array_equal(caches[0].codes[:, 13], c)
    assert np.array_equal(caches[0].scales[:, 13], s)
    assert r["idx"][0].shape == (2, 4)
    assert r["idx"][0][0].tolist() == [0, 1, -1, -1]


def test_malformed_stacks_rejected():
    caches = _caches(1, 1, 64)
    q = W.queries(0, 0, 0, 1, 2)
    with pytest.raises(ValueError):
        decode_step(caches, [(REUSE, 0, q)], None, 4, 0, 0.1)
    with pytest.raises(ValueError):
        decode_step(caches, [(REINDEX, 0, q)], None, 4, 0, 0.1)
    caches2 = _caches(2, 1, 64)
    with pytest.raises(ValueError):
        decode_step(caches2, [(FULL, 0, q), (FULL, 1, q), (REINDEX, 0, q)], None, 4, 0, 0.1)
    with pytest.raises(ValueError):
        Cache(1, 12)
