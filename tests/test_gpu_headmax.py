"""Per-head indexer score rule on the GPU against the oracle (score =
best head's pinned-order score): scores bit-exact, pools and selections
byte-equal, a decode step's indices byte-equal and outputs within the
attention bound.  Heads 1..64 cover the three lane layouts (16, 32 and 64
lanes per block) with lanes past the last head; ragged lengths cover partial
last blocks, tiles that straddle a sequence's end and empty sequences."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
import workloads as W
from oracle import indexer as I
from oracle.select import select
from oracle.step import FULL, REINDEX, REUSE, decode_step
from tests._gpu import ATT_TOL, cap_for, log, normwise_err, oracle_cache, require_gpu, to_device

pytestmark = pytest.mark.gpu

HM = I.SCORE_HEADMAX


def _scores_gpu(g, q, cand=None):
    B = g.batch
    width = (g.max_len + 7) // 8 if cand is None else cand.shape[1]
    out = torch.full((B, max(width, 1)), 7.0, dtype=torch.float32, device="cuda")
    csa2.block_scores(g, torch.from_numpy(q).cuda(), out,
                      cand=None if cand is None else torch.from_numpy(cand).cuda(), score=csa2.SCORE_HEADMAX)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("heads", [1, 5, 16, 17, 32, 33, 64])
def test_headmax_scores_bit_exact_ragged(heads):
    require_gpu()
    lengths = [2053, 8 * 37 + 5, 1, 0, 136]
    oc = oracle_cache(4, 0, lengths, cap_for(max(lengths)))
    g = to_device(oc)
    q = W.queries(4, 1, heads, len(lengths), heads)
    log(f"headmax scores: heads={heads} lengths={lengths}")
    got = _scores_gpu(g, q)
    assert csa2.device_error() == 0
    for b, n in enumerate(lengths):
        ids, want = I.block_scores(oc.codes[b], oc.scales[b], n, q[b], score=HM)
        nb = len(ids)
        assert got[b, :nb].tobytes() == want.tobytes(), (b, np.flatnonzero(got[b, :nb] != want)[:5])
        assert np.all(np.isneginf(got[b, nb:]))


def test_headmax_scores_candidates_and_bad_ids():
    """Candidate lists with -1 entries (-inf, no flag) and an id past the
    sequence's end (-inf, FLAG_BAD_INDEX)."""
    require_gpu()
    lengths = [3001, 2000]
    oc = oracle_cache(4, 1, lengths, cap_for(3001))
    g = to_device(oc)
    q = W.queries(4, 2, 0, 2, 64)
    rng = np.random.default_rng(3)
    cand = np.stack([rng.permutation(376)[:101], rng.permutation(250)[:101]]).astype(np.int32)
    cand[0, 7] = -1
    cand[1, 100] = -1
    got = _scores_gpu(g, q, cand)
    assert csa2.device_error() == 0
    for b, n in enumerate(lengths):
        ids, want = I.block_scores(oc.codes[b], oc.scales[b], n, q[b], cand=cand[b], score=HM)
        keep = cand[b] >= 0
        assert got[b][keep].tobytes() == want.tobytes()
        assert np.all(np.isneginf(got[b][~keep]))
    bad = cand.copy()
    bad[1, 3] = 250 + 4                                   # sequence 1 has 250 blocks
    got = _scores_gpu(g, q, bad)
    assert csa2.device_error() & csa2.FLAG_BAD_INDEX
    assert np.isneginf(got[1, 3])


def _index(g, q, topk, pool=0, cand=None, ws=None):
    B = g.batch
    ws = ws if ws is not None else csa2.workspace(B, q.shape[1], g.max_len, pool, topk)
    idx = torch.full((B, topk), -7, dtype=torch.int32, device="cuda")
    pool_out = torch.full((B, pool), -7, dtype=torch.int32, device="cuda") if pool else None
    csa2.index_topk(csa2.FULL, g, torch.from_numpy(q).cuda(), topk, idx, ws,
                    cand=None if cand is None else torch.from_numpy(cand).cuda(),
                    pool=pool, pool_out=pool_out, score=csa2.SCORE_HEADMAX)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (pool_out.cpu().numpy() if pool else None), ws


@pytest.mark.parametrize("lengths,heads,topk,pool", [
    ([4096], 64, 64, 0),
    ([4096, 1000, 9, 0], 16, 64, 0),
    ([40000 + 3, 16001], 64, 256, 2048),
    ([20000, 16], 32, 128, 2048),
])
def test_headmax_selection_matches_oracle(lengths, heads, topk, pool):
    require_gpu()
    oc = oracle_cache(4, 2, lengths, cap_for(max(lengths)))
    g = to_device(oc)
    q = W.queries(4, 3, heads, len(lengths), heads)
    log(f"headmax index: lengths={lengths} heads={heads} topk={topk} pool={pool}")
    idx, pool_out, ws = _index(g, q, topk, pool)
    for b, n in enumerate(lengths):
        ids, sc = I.block_scores(oc.codes[b], oc.scales[b], n, q[b], score=HM)
        if pool:
            assert np.array_equal(pool_out[b], select(ids, sc, pool)), b
        assert np.array_equal(idx[b], select(ids, sc, topk)), (b, idx[b][:10])
    idx2, _, _ = _index(g, q, topk, pool, ws=ws)           # the workspace is left clean
    assert np.array_equal(idx, idx2)


@pytest.mark.parametrize("n_cand", [2048, 8192])
def test_headmax_candidate_selection(n_cand):
    """A Reindex-style call on a candidate list (per-head rescoring, then the
    list's top-k in one workgroup per sequence)."""
    require_gpu()
    lengths = [70000, 66001]
    oc = oracle_cache(4, 3, lengths, cap_for(70000))
    g = to_device(oc)
    q0 = W.queries(4, 4, 0, 2, 64)
    _, pool_out, ws = _index(g, q0, 256, n_cand)
    q1 = W.queries(4, 5, 0, 2, 64)
    idx1, _, _ = _index(g, q1, 256, 0, cand=pool_out, ws=ws)
    for b, n in enumerate(lengths):
        ids, sc = I.block_scores(oc.codes[b], oc.scales[b], n, q1[b], cand=pool_out[b], score=HM)
        assert np.array_equal(idx1[b], select(ids, sc, 256)), b


@pytest.mark.parametrize("pool", [2048, 4096, 0])
def test_headmax_decode_step_matches_oracle(pool):
    """A 5-layer step [Full, Reindex, Reuse, Full, Reindex] over two caches
    with an append: indices byte-equal, outputs within the attention bound.
    pool 2,048: the top-k is taken inside the attention kernel; 4,096: the
    rescoring's own selection; 0: every selecting layer scans all blocks."""
    require_gpu()
    lengths, H, K = [30001, 17000], 64, 64
    n_after = [n + 1 for n in lengths]
    cap = cap_for(max(n_after))
    ocs = [oracle_cache(4, 10 + c, lengths, cap) for c in range(2)]
    rows = np.stack([W.append_rows(4, c, 0, 2) for c in range(2)])          # [2, B, 512]
    gs = [to_device(oc, max_len=max(n_after)) for oc in ocs]
    pattern = [(FULL, 0), (REINDEX, 0), (REUSE, 0), (FULL, 1), (REINDEX, 1)]
    qs = [W.queries(4, 20 + l, 0, 2, H) for l in range(len(pattern))]
    scale = 1.0 / np.sqrt(512.0)
    outs = [torch.zeros((2, H, 512), dtype=torch.float32, device="cuda") for _ in pattern]
    idxs = [torch.full((2, K), -9, dtype=torch.int32, device="cuda") for _ in pattern]
    layers = [(m, c, torch.from_numpy(qs[l]).cuda(), outs[l], idxs[l]) for l, (m, c) in enumerate(pattern)]
    pool_t = torch.full((2, pool), -9, dtype=torch.int32, device="cuda") if pool else None
    ws = csa2.workspace(2, H, max(n_after), pool, K)
    log(f"headmax decode step: pool={pool}")
    csa2.decode_step(gs, layers, H, K, pool, scale, ws, pool_out=pool_t,
                     new_rows=torch.from_numpy(rows).cuda(), score=csa2.SCORE_HEADMAX)
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    # oracle: the same append, the same layers
    ref = decode_step(ocs, [(m, c, qs[l]) for l, (m, c) in enumerate(pattern)], rows, K, pool, scale,
                      score=HM)
    if pool:
        assert np.array_equal(pool_t.cpu().numpy(), np.stack(ref["pool"]))
    for l in range(len(pattern)):
        assert np.array_equal(idxs[l].cpu().numpy(), np.stack(ref["idx"][l])), l
        assert normwise_err(outs[l].cpu().numpy(), np.stack(ref["out"][l])) <= ATT_TOL, l


def test_headmax_decode_step_noalloc_matches_workspace_step():
    """csa2_decode_step_noalloc carries the score rule like csa2_decode_step."""
    require_gpu()
    lengths, H, K, P = [9000], 32, 32, 512
    oc = oracle_cache(4, 30, lengths, cap_for(9000))
    q = [torch.from_numpy(W.queries(4, 40 + l, 0, 1, H)).cuda() for l in range(2)]
    res = []
    for noalloc in (False, True):
        g = to_device(oc)
        outs = [torch.zeros((1, H, 512), dtype=torch.float32, device="cuda") for _ in range(2)]
        idxs = [torch.full((1, K), -9, dtype=torch.int32, device="cuda") for _ in range(2)]
        layers = [(FULL, 0, q[0], outs[0], idxs[0]), (REINDEX, 0, q[1], outs[1], idxs[1])]
        pool = torch.full((1, P), -9, dtype=torch.int32, device="cuda")
        if noalloc:
            csa2.decode_step_noalloc([g], layers, H, K, P, 0.05, pool_out=pool, score=csa2.SCORE_HEADMAX)
        else:
            ws = csa2.workspace(1, H, g.max_len, P, K)
            csa2.decode_step([g], layers, H, K, P, 0.05, ws, pool_out=pool, score=csa2.SCORE_HEADMAX)
        torch.cuda.synchronize()
        res.append((pool.cpu().numpy(), [i.cpu().numpy() for i in idxs], [o.cpu().numpy() for o in outs]))
    assert np.array_equal(res[0][0], res[1][0])
    for l in range(2):
        assert np.array_equal(res[0][1][l], res[1][1][l])
        assert np.array_equal(res[0][2][l], res[1][2][l])
    ids, sc = I.block_scores(oc.codes[0], oc.scales[0], 9000, W.queries(4, 40, 0, 1, H)[0], score=HM)
    assert np.array_equal(res[0][0][0], select(ids, sc, P))


def test_headmax_nonfinite_query_flags():
    require_gpu()
    oc = oracle_cache(4, 31, [500], cap_for(500))
    g = to_device(oc)
    q = W.queries(4, 50, 0, 1, 16)
    q[0, 9, 300] = np.inf
    assert csa2.device_error() == 0
    _scores_gpu(g, q)
    assert csa2.device_error() & csa2.FLAG_NONFINITE_Q
