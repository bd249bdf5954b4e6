"""The synthetic workloads have the pages' shapes and are reproducible (CPU)."""
import numpy as np

import workloads as W


def test_shapes_match_descriptions(golden):
    w3 = W.WORKLOADS[3]
    assert w3.context == 2 ** 20 and w3.heads == 64 and w3.topk == 256
    assert w3.pool == golden["pool_blocks"] and len(w3.pattern) == 20 and w3.n_caches == 4
    assert w3.layer_caches() == [0, 0, 0, 0, 0, 1, 1, 1, 1, 1, 2, 2, 2, 2, 2, 3, 3, 3, 3, 3]
    w4 = W.WORKLOADS[4]
    L = W.lengths(w4)
    assert L.shape == (64,) and L.min() >= 32768 and L.max() <= 131072
    assert W.WORKLOADS[2].pool * 8 == golden["pool_positions"]


def test_rows_reproducible_and_chunk_independent():
    a = W.kv_rows(1, 0, 2, 65530, 12)
    b = W.kv_rows(1, 0, 2, 0, 65542)[65530:]
    assert np.array_equal(a, b)
    assert a.dtype == np.float32
    r = W.rotation(1)
    assert np.allclose(r @ r.T, np.eye(512), atol=1e-12)


def test_queries_and_appends_fresh_per_layer_and_step():
    q0 = W.queries(3, 0, 0, 1, 64)
    q1 = W.queries(3, 1, 0, 1, 64)
    q2 = W.queries(3, 0, 1, 1, 64)
    assert q0.shape == (1, 64, 512) and not np.array_equal(q0, q1) and not np.array_equal(q0, q2)
    a = W.append_rows(3, 0, 0, 2)
    assert a.shape == (2, 512)
