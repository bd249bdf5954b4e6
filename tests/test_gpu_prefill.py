"""GPU batched prefill-side sparse attention (csa2_prefill_attend) against
the oracle (oracle.prefill): every output within 2e-3 (normwise per head).
Cache bytes come from the oracle's quantiser; each query's selection is a
seeded random choice of blocks at or before its own block (its own,
possibly partial, block always included), -1 padded."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
import workloads as W
from oracle.prefill import prefill_attend
from tests._gpu import ATT_TOL, cap_for, log, normwise_err, oracle_cache, require_gpu, to_device

pytestmark = pytest.mark.gpu


def _selection(rng, qpos, topk):
    idx = np.full((len(qpos), topk), -1, dtype=np.int32)
    for t, p in enumerate(qpos):
        own = int(p) // 8
        avail = np.arange(own)
        k = min(topk - 1, avail.size)
        pick = rng.choice(avail, k, replace=False) if k else np.zeros(0, dtype=np.int64)
        sel = np.sort(np.concatenate([pick, [own]]))
        idx[t, :sel.size] = sel
    return idx


def _run(n, qpos, heads, topk, seed):
    require_gpu()
    rng = np.random.default_rng(seed)
    oc = oracle_cache(2, 0, [n], cap_for(n))
    g = to_device(oc)
    qpos = np.asarray(qpos, dtype=np.int64)
    T = qpos.size
    q = W.queries(2, 7, seed, T, heads)
    idx = _selection(rng, qpos, topk)
    scale = 1 / np.sqrt(512)
    out = torch.full((T, heads, 512), float("nan"), dtype=torch.float32, device="cuda")
    ws = csa2.prefill_workspace(T, heads, topk)
    csa2.prefill_attend(g, 0, torch.from_numpy(q).cuda(), torch.from_numpy(qpos).cuda(),
                        torch.from_numpy(idx).cuda(), scale, out, ws)
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    ref = prefill_attend(oc.codes[0], oc.scales[0], qpos, q, idx, scale)
    err = normwise_err(out.cpu().numpy(), ref)
    log(f"prefill T={T} H={heads} K={topk} (workspace {0 if ws is None else ws.numel()} B): error {err:.2e}")
    assert err <= ATT_TOL


def test_prefill_chunk_few_queries_split_k():
    # 5 queries of 64 heads: each query's selection is split over 32
    # workgroups (all four head tiles each) and merged
    n = 9000
    _run(n, [n - 5, n - 4, n - 3, n - 2, n - 1], 64, 256, 1)


def test_prefill_chunk_many_queries_two_splits():
    # 300 queries of 64 heads: two workgroups per query, merged
    n = 12000
    _run(n, np.arange(n - 300, n), 64, 256, 2)


def test_prefill_chunk_many_queries_one_split():
    # 520 queries of 64 heads: one workgroup per query normalises in-kernel
    n = 6000
    _run(n, np.sort(np.random.default_rng(9).choice(n, 520, replace=False)), 64, 40, 4)


def test_prefill_16_heads_many_queries_one_split():
    # 16 heads, 600 queries: the per-head-tile kernel with one split
    n = 5000
    _run(n, np.arange(n - 600, n), 16, 24, 5)


def test_prefill_ragged_positions_16_heads():
    # early queries with fewer blocks than topk (-1 padding), partial own blocks
    qpos = [0, 1, 7, 8, 63, 64, 200, 511, 1000, 4093, 4094, 4095]
    _run(4096, qpos, 16, 64, 3)


def test_prefill_32_heads_split_k():
    # 32 heads (two head tiles per query in the per-tile kernel), a few queries, split over workgroups
    n = 7000
    _run(n, [100, 3000, 6999, 6998, 5555, 17], 32, 128, 6)
