"""GPU indexer vs the oracle: block scores bit-exact, selected ids and pools
byte-equal (lowest-id tie-break), Reuse copies exactly."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
import workloads as W
from oracle import indexer as I
from oracle.select import select
from oracle.step import Cache
from tests._gpu import cap_for, log, oracle_cache, require_gpu, to_device

pytestmark = pytest.mark.gpu


def _scores_gpu(g, q, cand=None):
    B = g.batch
    if cand is None:
        nb = (g.max_len + 7) // 8
        out = torch.full((B, nb), 7.0, dtype=torch.float32, device="cuda")
    else:
        out = torch.full((B, cand.shape[1]), 7.0, dtype=torch.float32, device="cuda")
    csa2.block_scores(g, torch.from_numpy(q).cuda(), out,
                      cand=None if cand is None else torch.from_numpy(cand).cuda())
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("heads", [1, 16, 64])
def test_block_scores_bit_exact_ragged(heads):
    require_gpu()
    lengths = [4096, 4093, 17, 1, 0, 8 * 37 + 5]
    oc = oracle_cache(0, 0, lengths, cap_for(4096))
    g = to_device(oc)
    q = W.queries(0, 5, heads, len(lengths), heads)
    log(f"block scores: heads={heads} lengths={lengths}")
    got = _scores_gpu(g, q)
    for b, n in enumerate(lengths):
        ids, want = I.block_scores(oc.codes[b], oc.scales[b], n, q[b])
        nb = len(ids)
        assert got[b, :nb].tobytes() == want.tobytes(), (b, np.flatnonzero(got[b, :nb] != want)[:5])
        assert np.all(np.isneginf(got[b, nb:]))


def test_block_scores_candidates():
    require_gpu()
    lengths = [2000, 3001]
    oc = oracle_cache(0, 1, lengths, cap_for(3001))
    g = to_device(oc)
    q = W.queries(0, 6, 0, 2, 16)
    rng = np.random.default_rng(1)
    cand = np.stack([rng.permutation(250)[:100], rng.permutation(376)[:100]]).astype(np.int32)
    cand[0, 7] = -1
    got = _scores_gpu(g, q, cand)
    for b, n in enumerate(lengths):
        ids, want = I.block_scores(oc.codes[b], oc.scales[b], n, q[b], cand=cand[b])
        keep = cand[b] >= 0
        assert got[b][keep].tobytes() == want.tobytes()
        assert np.all(np.isneginf(got[b][~keep]))


def _index(g, q, topk, pool=0, cand=None, ws=None):
    B = g.batch
    ws = ws if ws is not None else csa2.workspace(B, q.shape[1], g.max_len, pool, topk)
    idx = torch.full((B, topk), -7, dtype=torch.int32, device="cuda")
    pool_out = torch.full((B, pool), -7, dtype=torch.int32, device="cuda") if pool else None
    csa2.index_topk(csa2.FULL, g, torch.from_numpy(q).cuda(), topk, idx, ws,
                    cand=None if cand is None else torch.from_numpy(cand).cuda(),
                    pool=pool, pool_out=pool_out)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (pool_out.cpu().numpy() if pool else None), ws


@pytest.mark.parametrize("lengths,topk,pool", [
    ([4096], 64, 0),                       # single Full layer, 4,096 positions, top-64
    ([4096, 1000, 9, 0], 64, 0),           # ragged batch, fewer blocks than k, empty
    ([65536 + 3], 256, 2048),              # pool + top-k inside it
    ([20000, 16000, 16], 128, 2048),       # pool larger than some sequences
    ([70000, 20001, 5], 256, 2048),        # ragged batch over several 4,096-block select workgroups
])
def test_full_scan_selection_matches_oracle(lengths, topk, pool):
    require_gpu()
    oc = oracle_cache(1, 0, lengths, cap_for(max(lengths)))
    g = to_device(oc)
    q = W.queries(1, 0, 0, len(lengths), 16)
    log(f"index: lengths={lengths} topk={topk} pool={pool}")
    idx, pool_out, ws = _index(g, q, topk, pool)
    for b, n in enumerate(lengths):
        ids, sc = I.block_scores(oc.codes[b], oc.scales[b], n, q[b])
        if pool:
            want_pool = select(ids, sc, pool)
            assert np.array_equal(pool_out[b], want_pool), b
            keep = np.isin(ids, want_pool)
            want = select(ids[keep], sc[keep], topk)
            assert np.array_equal(want, select(ids, sc, topk))      # nesting
        else:
            want = select(ids, sc, topk)
        assert np.array_equal(idx[b], want), (b, idx[b][:10], want[:10])
    # the workspace is left clean: a second call gives the same answer
    idx2, pool2, _ = _index(g, q, topk, pool, ws=ws)
    assert np.array_equal(idx, idx2)


def test_rescore_pool_candidates():
    require_gpu()
    lengths = [70000, 50001]
    oc = oracle_cache(2, 0, lengths, cap_for(70000))
    g = to_device(oc)
    q0 = W.queries(2, 0, 0, 2, 64)
    idx0, pool_out, ws = _index(g, q0, 256, 2048)
    q1 = W.queries(2, 1, 0, 2, 64)
    idx1, _, _ = _index(g, q1, 256, 0, cand=pool_out, ws=ws)
    for b, n in enumerate(lengths):
        ids, sc = I.block_scores(oc.codes[b], oc.scales[b], n, q1[b], cand=pool_out[b])
        assert np.array_equal(idx1[b], select(ids, sc, 256)), b


def test_ties_lowest_id_and_large_tie_bucket():
    """Every block identical: all scores tie, so the lowest ids win; with
    more blocks than fit the finisher's LDS the global path is used."""
    require_gpu()
    rows = W.kv_rows(0, 3, 0, 0, 8)
    for nblk in (300, 12000):
        oc = Cache(1, nblk * 8)
        for b0 in range(0, nblk, 1000):
            cnt = min(1000, nblk - b0)
            oc.write(0, 8 * b0, np.tile(rows, (cnt, 1)))
        oc.seq_len[0] = nblk * 8
        g = to_device(oc)
        q = W.queries(0, 7, 0, 1, 16)
        idx, pool_out, _ = _index(g, q, 64, 2048)
        assert pool_out[0].tolist() == list(range(min(2048, nblk))) + [-1] * max(0, 2048 - nblk)
        assert idx[0].tolist() == list(range(64))


@pytest.mark.parametrize("nblk,ntypes,pool,topk", [
    (20000, 5, 2048, 64),       # 4,000 blocks per score: the tie digit is ranked in LDS by id
    (30000, 3, 2048, 256),      # 10,000 tied blocks: more than the LDS list, digits re-counted from the scores
    (30000, 3, 0, 512),         # the same without a pool
    (270000, 5, 2048, 256),     # 270,000 blocks: the selection bitmap does not fit in LDS
])
def test_selection_with_repeated_block_types(nblk, ntypes, pool, topk):
    """Blocks drawn from a few distinct 8-row blocks, so whole score levels
    tie across the threshold: the lowest ids of the level win."""
    require_gpu()
    small = Cache(1, 8 * ntypes)
    small.write(0, 0, W.kv_rows(0, 3, 0, 0, 8 * ntypes))
    small.seq_len[0] = 8 * ntypes
    q = W.queries(0, 7, 0, 1, 16)
    _, type_score = I.block_scores(small.codes[0], small.scales[0], 8 * ntypes, q[0])
    ids = np.arange(nblk, dtype=np.int64)
    types = (ids * 7919 + 3) % ntypes
    scores = type_score[types]
    log(f"repeated blocks: nblk={nblk} types={ntypes} pool={pool} topk={topk}")
    g = csa2.KVCache(1, nblk * 8)
    tt = torch.from_numpy(types).cuda()
    g.codes[0].copy_(torch.from_numpy(small.codes[0].reshape(ntypes, 8, 256)).cuda()[tt].reshape(-1, 256))
    g.scales[0].copy_(torch.from_numpy(small.scales[0].reshape(ntypes, 8, 32)).cuda()[tt].reshape(-1, 32))
    g.seq_len.fill_(nblk * 8)
    g.max_len = nblk * 8
    del tt
    idx, pool_out, ws = _index(g, q, topk, pool)
    if pool:
        want_pool = select(ids, scores, pool)
        assert np.array_equal(pool_out[0], want_pool)
        keep = np.isin(ids, want_pool)
        want = select(ids[keep], scores[keep], topk)
    else:
        want = select(ids, scores, topk)
    assert np.array_equal(idx[0], want), (idx[0][:8], want[:8])
    idx2, _, _ = _index(g, q, topk, pool, ws=ws)
    assert np.array_equal(idx, idx2)


@pytest.mark.parametrize("batch", [512, 520])
def test_many_short_sequences(batch):
    """512 sequences take the batch scan over the chunks laid end to end;
    520 exceed its per-workgroup length table and take one scan per
    sequence.  Short ragged sequences (1..200 positions), top-4 and pool 16."""
    require_gpu()
    lengths = np.random.default_rng(batch).integers(1, 201, batch)
    # 8 source sequences quantised once by the oracle; sequence b holds the
    # first lengths[b] rows of source b % 8 (its own query keeps its choice
    # its own)
    src = Cache(8, 200)
    for k in range(8):
        src.write(k, 0, W.kv_rows(1, 2, k, 0, 200))
    oc = Cache(batch, cap_for(int(lengths.max())))
    for b, n in enumerate(lengths):
        oc.codes[b, :n] = src.codes[b % 8, :n]
        oc.scales[b, :n] = src.scales[b % 8, :n]
        oc.seq_len[b] = n
    g = to_device(oc)
    q = W.queries(1, 9, 0, batch, 4)
    log(f"many sequences: batch={batch}")
    ref = [I.block_scores(oc.codes[b], oc.scales[b], int(n), q[b]) for b, n in enumerate(lengths)]
    for pool in (0, 16):
        idx, pool_out, _ = _index(g, q, 4, pool)
        for b, (ids, sc) in enumerate(ref):
            if pool:
                assert np.array_equal(pool_out[b], select(ids, sc, pool)), b
            assert np.array_equal(idx[b], select(ids, sc, 4)), (b, pool)


def test_reuse_copies_prior():
    require_gpu()
    prior = torch.arange(3 * 40, dtype=torch.int32, device="cuda").view(3, 40)
    out = torch.full((3, 40), -5, dtype=torch.int32, device="cuda")
    csa2.index_topk(csa2.REUSE, None, None, 40, out, None, prior_idx=prior)
    torch.cuda.synchronize()
    assert torch.equal(out, prior)
