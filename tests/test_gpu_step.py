"""GPU layer-stack driver vs the oracle over whole decode steps: every
layer's selection (and the pool) byte-equal, every output within 2e-3.
The workloads keep their layer patterns, heads, top-k and pool; contexts
are cut so the oracle finishes in seconds (full sizes: test_gpu_fullsize)."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
import workloads as W
from oracle.step import decode_step as oracle_step
from tests._gpu import ATT_TOL, cap_for, log, normwise_err, oracle_cache, require_gpu, to_device
from tests.test_gpu_swa import oracle_swa, ring_to_device

pytestmark = pytest.mark.gpu


def run_and_compare(w, lengths, steps, window=0):
    """window > 0: every layer has a local branch (FP8 ring of that many
    positions, prefilled like the caches, one row appended per step)."""
    require_gpu()
    lengths = np.asarray(lengths, dtype=np.int64)
    B = len(lengths)
    cap = cap_for(int(lengths.max()), steps if w.append else 0)
    ocs = [oracle_cache(w.wid, c, lengths, cap) for c in range(w.n_caches)]
    gcs = [to_device(oc) for oc in ocs]
    caches_of = w.layer_caches()
    L = len(w.pattern)
    oswa = [oracle_swa(w.wid, l, lengths, window, int(lengths.max()) + steps) for l in range(L)] if window else None
    rings = [ring_to_device(o, window) for o in oswa] if window else None
    max_len = int(lengths.max()) + (steps if w.append else 0)
    ws = csa2.workspace(B, w.heads, max_len, w.pool, w.topk)
    pool_out = torch.zeros((B, w.pool), dtype=torch.int32, device="cuda") if w.pool else None
    for step in range(steps):
        qs = [W.queries(w.wid, l, step, B, w.heads) for l in range(L)]
        new_rows = np.stack([W.append_rows(w.wid, c, step, B) for c in range(w.n_caches)]) if w.append else None
        srows = np.stack([W.swa_append_rows(w.wid, l, step, B) for l in range(L)]) if window else None
        ref = oracle_step(ocs, [(m, caches_of[l], qs[l]) for l, m in enumerate(w.pattern)],
                          new_rows, w.topk, w.pool, w.scale, swa=oswa, swa_rows=srows, window=window)
        for g in gcs:
            g.max_len = int(lengths.max()) + ((step + 1) if w.append else 0)
        qt = [torch.from_numpy(q).cuda() for q in qs]
        outs = [torch.zeros((B, w.heads, 512), dtype=torch.float32, device="cuda") for _ in range(L)]
        idxs = [torch.full((B, w.topk), -9, dtype=torch.int32, device="cuda") for _ in range(L)]
        layers = [(m, caches_of[l], qt[l], outs[l], idxs[l]) for l, m in enumerate(w.pattern)]
        if window:
            st = [torch.from_numpy(srows[l]).cuda() for l in range(L)]
            layers = [ly + (rings[l], st[l]) for l, ly in enumerate(layers)]
        nr = torch.from_numpy(new_rows).cuda() if new_rows is not None else None
        csa2.decode_step(gcs, layers, w.heads, w.topk, w.pool, w.scale, ws, pool_out=pool_out, new_rows=nr)
        torch.cuda.synchronize()
        assert csa2.device_error() == 0
        for c, (g, oc) in enumerate(zip(gcs, ocs)):
            assert np.array_equal(g.seq_len.cpu().numpy(), oc.seq_len)
        if w.pool:
            assert np.array_equal(pool_out.cpu().numpy(), ref["pool"]), step
        worst = 0.0
        for l in range(L):
            gi = idxs[l].cpu().numpy()
            assert np.array_equal(gi, ref["idx"][l]), (step, l, w.pattern[l])
            err = normwise_err(outs[l].cpu().numpy(), ref["out"][l])
            worst = max(worst, err)
            assert err <= ATT_TOL, (step, l, err)
        if window:
            for l in range(L):
                assert np.array_equal(rings[l].seq_len.cpu().numpy(), oswa[l].seq_len)
        log(f"{w.name} step {step}: idx equal on {L} layers, worst attention error {worst:.2e}"
            + (f" (window {window})" if window else ""))


def test_workload0_single_full_4k():
    w = W.WORKLOADS[0]
    run_and_compare(w, [w.context], 1)


def test_workload1_full_reindex_reuse_b4():
    w = W.scaled(W.WORKLOADS[1], context=8192)
    run_and_compare(w, [8192] * 4, 1)


def test_workload2_hierarchical_pool():
    w = W.scaled(W.WORKLOADS[2], context=32768)
    run_and_compare(w, [32768], 1)


def test_workload3_twenty_layers_appending():
    w = W.scaled(W.WORKLOADS[3], context=20000)
    run_and_compare(w, [20000 - 3], 3)


def test_workload4_ragged_batch_appending():
    w = W.scaled(W.WORKLOADS[4], context=0, batch=6)
    lengths = np.random.default_rng(4).integers(4000, 20000, 6)
    run_and_compare(w, lengths, 2)


def test_pool_not_a_multiple_of_256():
    # in-attention top-k over a ragged candidate list (600 entries, 40 kept)
    w = W.scaled(W.WORKLOADS[3], context=12000, pool=600, topk=40)
    run_and_compare(w, [12000 - 2], 2)


def test_pool_above_in_kernel_limit():
    # a pool beyond 2,048 candidates takes the separate top-k kernels
    w = W.scaled(W.WORKLOADS[2], context=40000, pool=2600, topk=256)
    run_and_compare(w, [40000], 1)


def test_local_branch_twenty_layers_fused_selection():
    # every layer joins a 128-position FP8 window; pool <= 2,048 (top-k in the attention kernel)
    w = W.scaled(W.WORKLOADS[3], context=9000)
    run_and_compare(w, [9000 - 5], 2, window=128)


def test_local_branch_ragged_batch_separate_selection():
    # pool 0 (every selecting layer scans all blocks), ragged batch, window not a multiple of 64
    w = W.scaled(W.WORKLOADS[1], context=3000, batch=3)
    run_and_compare(w, [3000, 150, 1200], 2, window=200)


@pytest.mark.parametrize("ntypes,nblk", [
    (3, 24000),     # the pool holds one score level: every candidate ties (degenerate range)
    (8, 16000),     # two score levels, one holding 2,000 of the 2,048 candidates (crowded bin)
])
def test_tied_pool_scores_in_attention_selection(ntypes, nblk):
    """Blocks drawn from a few distinct 8-row blocks: the layer's top-k
    inside the pool (taken by the attention kernel) meets whole tied score
    levels, and the lowest ids of the level win."""
    from oracle.step import Cache, FULL, REINDEX, REUSE
    require_gpu()
    small = Cache(1, 8 * ntypes)
    small.write(0, 0, W.kv_rows(0, 3, 0, 0, 8 * ntypes))
    types = (np.arange(nblk, dtype=np.int64) * 7919 + 3) % ntypes
    oc = Cache(1, nblk * 8)
    oc.codes[0] = small.codes[0].reshape(ntypes, 8, 256)[types].reshape(-1, 256)
    oc.scales[0] = small.scales[0].reshape(ntypes, 8, 32)[types].reshape(-1, 32)
    oc.seq_len[0] = nblk * 8
    g = to_device(oc)
    H, K, P, scale = 64, 256, 2048, 1 / np.sqrt(512)
    pattern = (FULL, REINDEX, REUSE)
    qs = [W.queries(0, 20 + l, 0, 1, H) for l in range(len(pattern))]
    log(f"tied pool: types={ntypes} blocks={nblk}")
    ref = oracle_step([oc], [(m, 0, qs[l]) for l, m in enumerate(pattern)], None, K, P, scale)
    ws = csa2.workspace(1, H, nblk * 8, P, K)
    pool_out = torch.zeros((1, P), dtype=torch.int32, device="cuda")
    outs = [torch.zeros((1, H, 512), dtype=torch.float32, device="cuda") for _ in pattern]
    idxs = [torch.full((1, K), -9, dtype=torch.int32, device="cuda") for _ in pattern]
    layers = [(m, 0, torch.from_numpy(qs[l]).cuda(), outs[l], idxs[l]) for l, m in enumerate(pattern)]
    csa2.decode_step([g], layers, H, K, P, scale, ws, pool_out=pool_out)
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    assert np.array_equal(pool_out.cpu().numpy(), ref["pool"])
    for l in range(len(pattern)):
        assert np.array_equal(idxs[l].cpu().numpy(), ref["idx"][l]), l
        assert normwise_err(outs[l].cpu().numpy(), ref["out"][l]) <= ATT_TOL, l
