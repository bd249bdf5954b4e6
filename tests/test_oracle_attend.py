"""Pins for the oracle's sparse attention (CPU).

Pins: with every block selected it equals dense softmax attention computed
by torch's scaled_dot_product_attention (float64, a library routine); a
single position returns that row; identical rows return the row; positions
at or past n are masked; nothing selected gives zeros.
"""
import numpy as np
import torch

import workloads as W
from oracle import quantize as Q
from oracle.attend import gather_positions, sparse_attend


def _cache(n):
    return Q.quantize_rows(W.kv_rows(0, 0, 0, 0, n))


def test_all_blocks_equals_dense_attention():
    n = 8 * 20 + 3
    c, s = _cache(n)
    q = W.queries(0, 0, 0, 1, 16)[0]
    idx = np.arange(21, dtype=np.int32)
    out = sparse_attend(c, s, n, q, idx, 1 / np.sqrt(512))
    kv = torch.from_numpy(Q.dequantize_rows(c[:n], s[:n]).astype(np.float64))
    qt = torch.from_numpy(q.astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt[None, :, None, :], kv[None, None].expand(1, 16, n, 512), kv[None, None].expand(1, 16, n, 512),
        scale=1 / np.sqrt(512))[0, :, 0, :].numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_single_position_returns_row():
    n = 1
    c, s = _cache(8)
    q = W.queries(0, 1, 0, 1, 4)[0]
    out = sparse_attend(c, s, n, q, np.int32([0, -1]), 0.1)
    row = Q.dequantize_rows(c[:1], s[:1]).astype(np.float64)[0]
    assert np.array_equal(out, np.broadcast_to(row, out.shape))


def test_identical_rows_return_the_row():
    c, s = _cache(8)
    c = np.repeat(c[:1], 16, axis=0)
    s = np.repeat(s[:1], 16, axis=0)
    q = W.queries(0, 2, 0, 1, 4)[0]
    out = sparse_attend(c, s, 16, q, np.int32([1, 0]), 0.3)
    row = Q.dequantize_rows(c[:1], s[:1]).astype(np.float64)[0]
    assert np.allclose(out, row, rtol=0, atol=1e-12 * np.abs(row).max())


def test_positions_masked_at_n_and_empty():
    assert gather_positions([2, -1, 0], 19).tolist() == [16, 17, 18, 0, 1, 2, 3, 4, 5, 6, 7]
    c, s = _cache(24)
    q = W.queries(0, 3, 0, 1, 2)[0]
    assert np.all(sparse_attend(c, s, 0, q, np.int32([-1, -1]), 0.1) == 0)
    # garbage beyond n must not matter
    c2, s2 = c.copy(), s.copy()
    c2[19:] = 0x77
    s2[19:] = 0x70
    a = sparse_attend(c, s, 19, q, np.int32([2, 0]), 0.1)
    b = sparse_attend(c2, s2, 19, q, np.int32([2, 0]), 0.1)
    assert np.array_equal(a, b)
