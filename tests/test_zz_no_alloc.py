"""csa2_decode_step_noalloc (the library's own per-device workspace, for
callers that cannot allocate) against csa2_decode_step with a caller
workspace: two calls in a row, the second on a smaller step.  Same inputs on
both sides (the caches cloned before each step, since a step appends):
every layer's selection and the pool byte-equal, outputs within 2e-3 (the
kernels are the same, so they are in fact identical)."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
import workloads as W
from tests._gpu import ATT_TOL, log, normwise_err, require_gpu

pytestmark = pytest.mark.gpu


def _caches(wid, n_caches, lengths, cap):
    out = []
    for c in range(n_caches):
        g = csa2.KVCache(len(lengths), cap)
        for b, n in enumerate(lengths):
            x = torch.from_numpy(W.kv_rows(wid, c, b, 0, int(n))).cuda()
            csa2.fp4_quantize_kv(x, g.codes[b, :int(n)], g.scales[b, :int(n)])
        g.seq_len.copy_(torch.as_tensor(lengths, dtype=torch.int64))
        g.max_len = int(max(lengths)) + 1
        out.append(g)
    return out


def _clone(caches):
    out = []
    for g in caches:
        h = csa2.KVCache(g.batch, g.capacity)
        h.codes.copy_(g.codes)
        h.scales.copy_(g.scales)
        h.seq_len.copy_(g.seq_len)
        h.max_len = g.max_len
        out.append(h)
    return out


def _step(caches, pattern, heads, topk, pool, wid, noalloc):
    B = caches[0].batch
    lc, cur = [], -1
    for m in pattern:
        cur += 1 if m == csa2.FULL else 0
        lc.append(cur)
    qs = [torch.from_numpy(W.queries(wid, l, 0, B, heads)).cuda() for l in range(len(pattern))]
    outs = [torch.full((B, heads, 512), 5.0, dtype=torch.float32, device="cuda") for _ in pattern]
    idxs = [torch.full((B, topk), -9, dtype=torch.int32, device="cuda") for _ in pattern]
    pool_out = torch.full((B, pool), -9, dtype=torch.int32, device="cuda") if pool else None
    rows = torch.from_numpy(np.stack([W.append_rows(wid, c, 0, B) for c in range(len(caches))])).cuda()
    layers = [(m, lc[l], qs[l], outs[l], idxs[l]) for l, m in enumerate(pattern)]
    if noalloc:
        csa2.decode_step_noalloc(caches, layers, heads, topk, pool, 1 / np.sqrt(512), pool_out=pool_out,
                                 new_rows=rows)
    else:
        ws = csa2.workspace(B, heads, caches[0].max_len, pool, topk)
        csa2.decode_step(caches, layers, heads, topk, pool, 1 / np.sqrt(512), ws, pool_out=pool_out, new_rows=rows)
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    return ([i.cpu().numpy() for i in idxs], [o.cpu().numpy() for o in outs],
            None if pool_out is None else pool_out.cpu().numpy())


def test_noalloc_matches_workspace_step_twice():
    require_gpu()
    cases = [(2, [40000, 33001], (0, 1, 2, 1), 64, 256, 2048),
             (0, [9000], (0, 2), 16, 64, 0)]
    for wid, lengths, pattern, heads, topk, pool in cases:
        log(f"noalloc step: lengths {lengths}, pattern {pattern}, {heads} heads, top-{topk}, pool {pool}")
        n_caches = sum(1 for m in pattern if m == csa2.FULL)
        base = _caches(wid, n_caches, lengths, (max(lengths) + 8 + 7) // 8 * 8)
        ref = _step(_clone(base), pattern, heads, topk, pool, wid, noalloc=False)
        got = _step(_clone(base), pattern, heads, topk, pool, wid, noalloc=True)
        for l in range(len(pattern)):
            assert np.array_equal(got[0][l], ref[0][l]), l
            assert normwise_err(got[1][l], ref[1][l]) <= ATT_TOL, l
            assert np.array_equal(got[1][l], ref[1][l]), l
        if pool:
            assert np.array_equal(got[2], ref[2])
