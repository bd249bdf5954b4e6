"""Pins for the oracle's batched prefill-side sparse attention (CPU).

Pins: one query at the end of the cache is the decode attention; with every
block selected the outputs equal causal dense attention computed by torch's
scaled_dot_product_attention with a boolean mask (float64, a library
routine); rows after a query's position never change its output; queries
are independent (permuting them permutes the outputs).
"""
import numpy as np
import torch

import workloads as W
from oracle import quantize as Q
from oracle.attend import sparse_attend
from oracle.prefill import prefill_attend


def _cache(n):
    return Q.quantize_rows(W.kv_rows(0, 0, 0, 0, n))


def test_one_query_at_the_end_is_the_decode_attention():
    n = 8 * 9 + 5
    c, s = _cache(n)
    q = W.queries(0, 0, 0, 1, 16)
    idx = np.int32([[1, 4, 9, -1]])
    got = prefill_attend(c, s, [n - 1], q, idx, 0.07)
    want = sparse_attend(c, s, n, q[0], idx[0], 0.07)
    assert np.array_equal(got[0], want)


def test_all_blocks_equals_causal_dense_attention():
    n = 8 * 12 + 3
    c, s = _cache(n)
    T, H = 6, 8
    qpos = np.int64([0, 7, 8, 40, 77, n - 1])
    q = W.queries(0, 1, 0, T, H)
    nblk = (n + 7) // 8
    idx = np.tile(np.arange(nblk, dtype=np.int32), (T, 1))
    got = prefill_attend(c, s, qpos, q, idx, 1 / np.sqrt(512))
    kv = torch.from_numpy(Q.dequantize_rows(c[:n], s[:n]).astype(np.float64))
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]      # [1, H, T, 512]
    mask = torch.from_numpy(np.arange(n)[None, :] <= qpos[:, None])          # [T, n]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kv[None, None].expand(1, H, n, 512), kv[None, None].expand(1, H, n, 512),
        attn_mask=mask[None, None], scale=1 / np.sqrt(512))[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_causal_and_independent():
    n = 8 * 10
    c, s = _cache(n)
    T = 5
    qpos = np.int64([3, 20, 33, 50, 79])
    q = W.queries(0, 2, 0, T, 4)
    idx = np.int32([[0, -1, -1], [0, 2, -1], [1, 3, 4], [2, 5, 6], [0, 6, 9]])
    got = prefill_attend(c, s, qpos, q, idx, 0.05)
    # rows after every query's position do not matter to it
    for t in range(T):
        c2, s2 = c.copy(), s.copy()
        c2[qpos[t] + 1:] = 0x5A
        s2[qpos[t] + 1:] = 0x38
        assert np.array_equal(prefill_attend(c2, s2, qpos[t:t + 1], q[t:t + 1], idx[t:t + 1], 0.05)[0], got[t])
    perm = np.array([3, 0, 4, 1, 2])
    assert np.array_equal(prefill_attend(c, s, qpos[perm], q[perm], idx[perm], 0.05), got[perm])


def test_local_branch_query_is_the_decode_step_with_window():
    # each prefill query with a window equals the decode-step oracle with the
    # same window over a sequence that ends at the query's position
    from oracle import swa as S
    n, win = 8 * 11 + 3, 20
    c, s = _cache(n)
    sc, ss = S.quantize_fp8_rows(W.swa_rows(0, 3, 0, 0, n))
    qpos = np.int64([0, 5, 19, 20, 50, n - 1])
    q = W.queries(0, 4, 0, qpos.size, 16)
    idx = np.tile(np.int32([0, 3, 9, -1]), (qpos.size, 1))
    got = prefill_attend(c, s, qpos, q, idx, 0.06, sc, ss, win)
    for t, p in enumerate(qpos):
        want = S.attend_with_window(c, s, int(p) + 1, q[t], idx[t], 0.06, sc, ss, int(p) + 1, win)
        assert np.array_equal(got[t], want)
    # a window of 0 is the plain prefill attention
    assert np.array_equal(prefill_attend(c, s, qpos, q, idx, 0.06, sc, ss, 0), prefill_attend(c, s, qpos, q, idx, 0.06))
