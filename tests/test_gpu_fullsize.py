"""Full-size parity of the 20-layer decoder at 1,048,576 positions and of
the ragged batch-64 workload, in the launch configuration bench.py times
(GPU-quantised caches, one decode step through csa2_decode_step with the
Reuse layers sharing their predecessor's index buffer).

Expected values come from tests/golden/make_fullsize.py, which runs only the
CPU oracle on the same seeded inputs:
  * selection: the pool and every layer's selected blocks byte-equal to the
    oracle's;
  * scores: every full-scan score and every layer's pool scores bit-equal
    (sha256 of the float32 arrays the library exports against the oracle's);
  * bytes: the appended rows and sampled prefill rows equal the oracle's
    quantisation of the same synthetic rows;
  * attention: sampled layers' outputs against the oracle's float64
    attention over the selected positions (rows regenerated and quantised by
    the oracle), within the 2e-3 normwise bound.
The selections are also checked against the exported scores by the defining
property (every chosen key beats every other key, ties to the lowest id).
"""
import hashlib
import os

import numpy as np
import pytest
import torch

import bench
import fp4_compressed_sparse_amd as csa2
import workloads as W
from oracle.attend import gather_positions, sparse_attend
from oracle.indexer import block_keys, block_scores_from_keys, collapse_query
from oracle.quantize import quantize_rows
from tests._gpu import ATT_TOL, log, normwise_err, require_gpu

pytestmark = pytest.mark.gpu

BLOCK = 8
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with np.load(os.path.join(GOLDEN, name), allow_pickle=False) as z:
        return {k: z[k] for k in z.files}


def _sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


_CHUNKS = {}


def _chunks(wid, cache, chunk_ids):
    """Synthetic prefill chunks of one cache (kept for reuse), drawn on a
    thread pool: each chunk has its own seed."""
    from concurrent.futures import ThreadPoolExecutor
    need = [c for c in sorted(set(chunk_ids)) if (wid, cache, c) not in _CHUNKS]
    with ThreadPoolExecutor(max_workers=8) as ex:
        for c, rows in zip(need, ex.map(lambda c: W._kv_chunk(wid, cache, 0, c), need)):
            _CHUNKS[(wid, cache, c)] = rows
    return {c: _CHUNKS[(wid, cache, c)] for c in chunk_ids}


def _rows(wid, cache, positions, n_prefill, step_rows):
    """Synthetic float32 rows at the given positions of one cache: prefill
    rows from their chunks, position n_prefill is the step's appended row."""
    positions = np.asarray(positions, dtype=np.int64)
    out = np.empty((positions.size, 512), dtype=np.float32)
    pre = positions[positions != n_prefill]
    chunks = _chunks(wid, cache, (pre // W.CHUNK).tolist())
    for i, p in enumerate(positions.tolist()):
        out[i] = step_rows[cache] if p == n_prefill else chunks[p // W.CHUNK][p % W.CHUNK]
    return out


def _oracle_scores(wid, cache, blocks, n, n_prefill, step_rows, qbar):
    """Oracle scores of the given blocks (each block's rows quantised by the
    oracle, its key and pinned-order score computed on its own)."""
    out = []
    for beta in np.asarray(blocks).tolist():
        cnt = min(BLOCK, n - BLOCK * beta)
        pos = np.arange(BLOCK * beta, BLOCK * beta + cnt)
        codes, scales = quantize_rows(_rows(wid, cache, pos, n_prefill, step_rows))
        key = block_keys(codes, scales, cnt)
        out.append(block_scores_from_keys(qbar, key)[0])
    return np.asarray(out, dtype=np.float32)


def _top_keys_ok(ids, scores, chosen):
    """chosen (ascending ids) are exactly the top len(chosen) of (ids, scores)
    by (score descending, id ascending)."""
    ids = np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -scores.astype(np.float64)))
    want = np.sort(ids[order[:len(chosen)]])
    return np.array_equal(want, np.asarray(chosen, dtype=np.int64))


def test_decoder20_1m_full_size():
    require_gpu()
    _CHUNKS.clear()
    w = W.WORKLOADS[3]
    n0 = int(w.context)
    n = n0 + 1                                       # after this step's append
    cap = (n + 7) // 8 * 8
    rng = np.random.default_rng(20)
    log(f"building 4 caches of {n0} positions")
    caches = bench.build_caches(w, np.array([n0]), cap, log_every=1000)
    for c in caches:
        c.max_len = n
    L, H, K, P = len(w.pattern), w.heads, w.topk, w.pool
    lc = w.layer_caches()
    qs = [W.queries(w.wid, l, 0, 1, H) for l in range(L)]
    step_rows = np.stack([W.append_rows(w.wid, c, 0, 1) for c in range(w.n_caches)])   # [4, 1, 512]
    qt = [torch.from_numpy(q).cuda() for q in qs]
    outs = [torch.zeros((1, H, 512), dtype=torch.float32, device="cuda") for _ in range(L)]
    idxs = []
    for m in w.pattern:
        idxs.append(idxs[-1] if m == 2 else torch.full((1, K), -9, dtype=torch.int32, device="cuda"))
    pool = torch.full((1, P), -9, dtype=torch.int32, device="cuda")
    ws = csa2.workspace(1, H, n, P, K)
    layers = [(m, lc[l], qt[l], outs[l], idxs[l]) for l, m in enumerate(w.pattern)]
    csa2.decode_step(caches, layers, H, K, P, w.scale, ws, pool_out=pool,
                     new_rows=torch.from_numpy(step_rows).cuda())
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    log("decode step done")

    # appended rows and sampled prefill rows: bytes equal the oracle's
    for c, g in enumerate(caches):
        assert int(g.seq_len[0]) == n
        oc, osc = quantize_rows(step_rows[c])
        assert np.array_equal(g.codes[0, n0].cpu().numpy(), oc[0])
        assert np.array_equal(g.scales[0, n0].cpu().numpy(), osc[0])
    samp = np.sort(rng.choice(np.arange(0, 2 * W.CHUNK), 48, replace=False))
    oc, osc = quantize_rows(_rows(w.wid, 0, samp, n0, step_rows[:, 0]))
    assert np.array_equal(caches[0].codes[0, samp].cpu().numpy(), oc)
    assert np.array_equal(caches[0].scales[0, samp].cpu().numpy(), osc)
    log("appended and sampled rows byte-equal")

    gold = _golden("fullsize_decoder20_1m.npz")
    nblk = (n + BLOCK - 1) // BLOCK
    p = pool.cpu().numpy()[0]
    assert np.array_equal(p, gold["pool"]), "pool differs from the oracle's"
    for l in range(L):
        assert np.array_equal(idxs[l].cpu().numpy()[0], gold["idx"][l]), f"layer {l}: selection differs"
    log(f"pool ({P} blocks) and all {L} selections byte-equal to the oracle's")

    # full scan: all exported scores bit-equal to the oracle's
    s0 = torch.zeros((1, nblk), dtype=torch.float32, device="cuda")
    csa2.block_scores(caches[lc[0]], qt[0], s0)
    s0 = s0.cpu().numpy()[0]
    assert _sha(s0) == str(gold["scan_sha"]), "full-scan scores differ from the oracle's"
    assert _top_keys_ok(np.arange(nblk), s0, p)
    log(f"full scan: all {nblk} scores bit-equal to the oracle's")

    # every selecting layer's pool scores bit-equal; its top-K the top of them
    pool_t = pool.clone()
    prev = None
    for l, m in enumerate(w.pattern):
        got = idxs[l].cpu().numpy()[0]
        if m == 2:
            assert np.array_equal(got, prev), l
            continue
        sl = torch.zeros((1, P), dtype=torch.float32, device="cuda")
        csa2.block_scores(caches[lc[l]], qt[l], sl, cand=pool_t)
        sl = sl.cpu().numpy()[0]
        if l > 0:
            assert _sha(sl) == str(gold["pool_sha"][l]), f"layer {l}: pool scores differ"
        assert _top_keys_ok(p, sl, got), l
        prev = got
    log("every layer's pool scores bit-equal; selections are the top of them")

    # attention of a Full, a Reindex, a Reuse and the last layer against the
    # oracle (float64)
    for l in (0, 1, 2, L - 1):
        idx = idxs[l].cpu().numpy()[0]
        pos = gather_positions(idx, n)
        codes, scales = quantize_rows(_rows(w.wid, lc[l], pos, n0, step_rows[:, 0]))
        # compact cache: selected blocks in ascending order, the partial last
        # block (if chosen) last, so the compact length masks it the same way
        kept = idx[idx >= 0]
        ccodes = np.zeros((BLOCK * kept.size, 256), dtype=np.uint8)
        cscales = np.zeros((BLOCK * kept.size, 32), dtype=np.uint8)
        ccodes[:pos.size] = codes
        cscales[:pos.size] = scales
        ref = sparse_attend(ccodes, cscales, pos.size, qs[l][0], np.arange(kept.size), w.scale)
        err = normwise_err(outs[l].cpu().numpy()[0][None], ref[None])
        log(f"layer {l}: attention error {err:.2e} over {pos.size} positions")
        assert err <= ATT_TOL, (l, err)
    _CHUNKS.clear()


def test_decoder20_1m_full_size_per_head_rule():
    """The 20-layer step at 1,048,576 positions with the per-head score rule,
    in bench.py's launch configuration: the pool and all 20 selections
    byte-equal to the oracle's, the full scan's per-head scores and every
    pool layer's scores bit-equal (sha256), and two layers' attention
    against the oracle."""
    require_gpu()
    _CHUNKS.clear()
    w = W.WORKLOADS[3]
    n0 = int(w.context)
    n = n0 + 1
    cap = (n + 7) // 8 * 8
    log(f"building 4 caches of {n0} positions (per-head rule)")
    caches = bench.build_caches(w, np.array([n0]), cap, log_every=1000)
    for c in caches:
        c.max_len = n
    L, H, K, P = len(w.pattern), w.heads, w.topk, w.pool
    lc = w.layer_caches()
    qs = [W.queries(w.wid, l, 0, 1, H) for l in range(L)]
    step_rows = np.stack([W.append_rows(w.wid, c, 0, 1) for c in range(w.n_caches)])
    qt = [torch.from_numpy(q).cuda() for q in qs]
    outs = [torch.zeros((1, H, 512), dtype=torch.float32, device="cuda") for _ in range(L)]
    idxs = []
    for m in w.pattern:
        idxs.append(idxs[-1] if m == 2 else torch.full((1, K), -9, dtype=torch.int32, device="cuda"))
    pool = torch.full((1, P), -9, dtype=torch.int32, device="cuda")
    ws = csa2.workspace(1, H, n, P, K)
    layers = [(m, lc[l], qt[l], outs[l], idxs[l]) for l, m in enumerate(w.pattern)]
    csa2.decode_step(caches, layers, H, K, P, w.scale, ws, pool_out=pool,
                     new_rows=torch.from_numpy(step_rows).cuda(), score=csa2.SCORE_HEADMAX)
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    gold = _golden("fullsize_decoder20_1m_headmax.npz")
    nblk = (n + BLOCK - 1) // BLOCK
    p = pool.cpu().numpy()[0]
    assert np.array_equal(p, gold["pool"]), "pool differs from the oracle's"
    for l in range(L):
        assert np.array_equal(idxs[l].cpu().numpy()[0], gold["idx"][l]), f"layer {l}: selection differs"
    log(f"per-head rule: pool and all {L} selections byte-equal to the oracle's")
    s0 = torch.zeros((1, nblk), dtype=torch.float32, device="cuda")
    csa2.block_scores(caches[lc[0]], qt[0], s0, score=csa2.SCORE_HEADMAX)
    s0 = s0.cpu().numpy()[0]
    assert _sha(s0) == str(gold["scan_sha"]), "per-head full-scan scores differ from the oracle's"
    pool_t = pool.clone()
    for l, m in enumerate(w.pattern):
        if l == 0 or m == 2:
            continue
        sl = torch.zeros((1, P), dtype=torch.float32, device="cuda")
        csa2.block_scores(caches[lc[l]], qt[l], sl, cand=pool_t, score=csa2.SCORE_HEADMAX)
        assert _sha(sl.cpu().numpy()[0]) == str(gold["pool_sha"][l]), f"layer {l}: pool scores differ"
    log(f"per-head rule: all {nblk} scan scores and every layer's pool scores bit-equal")
    for l in (1, L - 1):
        idx = idxs[l].cpu().numpy()[0]
        pos = gather_positions(idx, n)
        codes, scales = quantize_rows(_rows(w.wid, lc[l], pos, n0, step_rows[:, 0]))
        kept = idx[idx >= 0]
        ccodes = np.zeros((BLOCK * kept.size, 256), dtype=np.uint8)
        cscales = np.zeros((BLOCK * kept.size, 32), dtype=np.uint8)
        ccodes[:pos.size] = codes
        cscales[:pos.size] = scales
        ref = sparse_attend(ccodes, cscales, pos.size, qs[l][0], np.arange(kept.size), w.scale)
        err = normwise_err(outs[l].cpu().numpy()[0][None], ref[None])
        log(f"layer {l}: attention error {err:.2e} over {pos.size} positions")
        assert err <= ATT_TOL, (l, err)
    _CHUNKS.clear()


def test_decoder20_1m_full_size_with_local_branch():
    """The same 20-layer step at 1,048,576 positions with a 128-position FP8
    window on every layer (ring bytes from the oracle's quantiser): the
    appended SWA rows are bit-equal to the oracle's, the selections are the
    top of their pool scores as before, and two layers' outputs match the
    oracle's joint softmax over the selected and the window positions."""
    from oracle import swa as S
    require_gpu()
    _CHUNKS.clear()
    w = W.WORKLOADS[3]
    n0 = int(w.context)
    n = n0 + 1
    cap = (n + 7) // 8 * 8
    win = 128
    log(f"building 4 caches of {n0} positions and 20 rings of {win}")
    caches = bench.build_caches(w, np.array([n0]), cap, log_every=1000)
    for c in caches:
        c.max_len = n
    L, H, K, P = len(w.pattern), w.heads, w.topk, w.pool
    lc = w.layer_caches()
    rings, wrows = [], []
    for l in range(L):
        rows = W.swa_rows(w.wid, l, 0, n0 - win, win)                 # positions n0-win .. n0-1
        c8, s8 = S.quantize_fp8_rows(rows)
        ring = csa2.SwaCache(1, win)
        slots = np.arange(n0 - win, n0) % win
        codes = np.zeros((win, 512), dtype=np.uint8)
        scales = np.zeros(win, dtype=np.float32)
        codes[slots], scales[slots] = c8, s8
        ring.codes[0].copy_(torch.from_numpy(codes))
        ring.scales[0].copy_(torch.from_numpy(scales))
        ring.seq_len.fill_(n0)
        rings.append(ring)
        wrows.append(rows)
    qs = [W.queries(w.wid, l, 0, 1, H) for l in range(L)]
    step_rows = np.stack([W.append_rows(w.wid, c, 0, 1) for c in range(w.n_caches)])
    srows = np.stack([W.swa_append_rows(w.wid, l, 0, 1) for l in range(L)])   # [L, 1, 512]
    qt = [torch.from_numpy(q).cuda() for q in qs]
    outs = [torch.zeros((1, H, 512), dtype=torch.float32, device="cuda") for _ in range(L)]
    idxs = []
    for m in w.pattern:
        idxs.append(idxs[-1] if m == 2 else torch.full((1, K), -9, dtype=torch.int32, device="cuda"))
    pool = torch.full((1, P), -9, dtype=torch.int32, device="cuda")
    ws = csa2.workspace(1, H, n, P, K)
    st = [torch.from_numpy(srows[l]).cuda() for l in range(L)]
    layers = [(m, lc[l], qt[l], outs[l], idxs[l], rings[l], st[l]) for l, m in enumerate(w.pattern)]
    csa2.decode_step(caches, layers, H, K, P, w.scale, ws, pool_out=pool,
                     new_rows=torch.from_numpy(step_rows).cuda())
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    log("decode step with local branch done")

    for l in range(L):
        assert int(rings[l].seq_len[0]) == n
        c8, s8 = S.quantize_fp8_rows(srows[l])
        assert np.array_equal(rings[l].codes[0, n0 % win].cpu().numpy(), c8[0])
        assert rings[l].scales[0, n0 % win].item() == s8[0]
    log("appended SWA rows bit-equal")

    p = pool.cpu().numpy()[0]
    gold = _golden("fullsize_decoder20_1m.npz")
    assert np.array_equal(p, gold["pool"]), "pool differs from the oracle's"
    for l in range(L):
        assert np.array_equal(idxs[l].cpu().numpy()[0], gold["idx"][l]), f"layer {l}: selection differs"
    log("pool and all selections byte-equal to the oracle's (the window does not change them)")
    pool_t = pool.clone()
    for l, m in enumerate(w.pattern):
        if m == 2:
            assert np.array_equal(idxs[l].cpu().numpy(), idxs[l - 1].cpu().numpy())
            continue
        sl = torch.zeros((1, P), dtype=torch.float32, device="cuda")
        csa2.block_scores(caches[lc[l]], qt[l], sl, cand=pool_t)
        assert _top_keys_ok(p, sl.cpu().numpy()[0], idxs[l].cpu().numpy()[0]), l

    for l in (0, L - 1):
        idx = idxs[l].cpu().numpy()[0]
        pos = gather_positions(idx, n)
        codes, scales = quantize_rows(_rows(w.wid, lc[l], pos, n0, step_rows[:, 0]))
        kept = idx[idx >= 0]
        ccodes = np.zeros((BLOCK * kept.size, 256), dtype=np.uint8)
        cscales = np.zeros((BLOCK * kept.size, 32), dtype=np.uint8)
        ccodes[:pos.size] = codes
        cscales[:pos.size] = scales
        # the window by position: n0-win+1 .. n0 (the appended row last)
        wc, wsc = S.quantize_fp8_rows(np.concatenate([wrows[l][1:], srows[l]], axis=0))
        ref = S.attend_with_window(ccodes, cscales, pos.size, qs[l][0], np.arange(kept.size), w.scale,
                                   wc, wsc, win, win)
        err = normwise_err(outs[l].cpu().numpy()[0][None], ref[None])
        log(f"layer {l}: attention with window error {err:.2e} over {pos.size} + {win} positions")
        assert err <= ATT_TOL, (l, err)
    _CHUNKS.clear()


def _seq_rows(wid, cache, b, positions, n0, step_row):
    """Synthetic float32 rows of sequence b at the given positions; position
    n0 is the step's appended row."""
    positions = np.asarray(positions, dtype=np.int64)
    out = np.empty((positions.size, 512), dtype=np.float32)
    chunks = {c: W._kv_chunk(wid, cache, b, c) for c in sorted(set((positions[positions != n0] // W.CHUNK).tolist()))}
    for i, p in enumerate(positions.tolist()):
        out[i] = step_row if p == n0 else chunks[p // W.CHUNK][p % W.CHUNK]
    return out


def test_workload4_ragged_batch64_full_size():
    """The batch workload at full size: 64 sequences of 32,768..131,072
    positions (seeded lengths), [Full, Reindex, Reuse], 16 heads, pool 2,048,
    top-128, one appended row each, in the launch configuration bench.py
    times (the batch scan over the sequences' chunks laid end to end).
    Checks: appended rows byte-equal the oracle's; every pool and every
    layer's selection byte-equal to the oracle's; every sequence's full-scan
    and Reindex pool scores bit-equal to the oracle's (and the selections the
    top of them); sampled scores recomputed block by block; attention of
    sampled sequences within 2e-3."""
    require_gpu()
    w = W.WORKLOADS[4]
    lengths = W.lengths(w)
    B = len(lengths)
    n = lengths + 1
    cap = int((int(n.max()) + 7) // 8 * 8)
    log(f"building the cache: {B} sequences of {int(lengths.min())}..{int(lengths.max())} positions")
    g = bench.build_caches(w, lengths, cap, log_every=1000)[0]
    g.max_len = int(n.max())
    H, K, P = w.heads, w.topk, w.pool
    L = len(w.pattern)
    qs = [W.queries(w.wid, l, 0, B, H) for l in range(L)]
    step_rows = W.append_rows(w.wid, 0, 0, B)                          # [B, 512]
    qt = [torch.from_numpy(q).cuda() for q in qs]
    outs = [torch.zeros((B, H, 512), dtype=torch.float32, device="cuda") for _ in range(L)]
    idxs = []
    for m in w.pattern:
        idxs.append(idxs[-1] if m == 2 else torch.full((B, K), -9, dtype=torch.int32, device="cuda"))
    pool = torch.full((B, P), -9, dtype=torch.int32, device="cuda")
    ws = csa2.workspace(B, H, g.max_len, P, K)
    layers = [(m, 0, qt[l], outs[l], idxs[l]) for l, m in enumerate(w.pattern)]
    csa2.decode_step([g], layers, H, K, P, w.scale, ws, pool_out=pool,
                     new_rows=torch.from_numpy(step_rows[None]).cuda())
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    log("decode step done")

    assert np.array_equal(g.seq_len.cpu().numpy(), n)
    oc, osc = quantize_rows(step_rows)
    for b in range(B):
        assert np.array_equal(g.codes[b, int(lengths[b])].cpu().numpy(), oc[b])
        assert np.array_equal(g.scales[b, int(lengths[b])].cpu().numpy(), osc[b])
    log("appended rows byte-equal")

    gold = _golden("fullsize_ragged_b64.npz")
    assert np.array_equal(gold["lengths"], lengths)
    p = pool.cpu().numpy()
    assert np.array_equal(p, gold["pool"]), "pools differ from the oracle's"
    for l in range(L):
        assert np.array_equal(idxs[l].cpu().numpy(), gold["idx"][l]), f"layer {l}: selections differ"
    log(f"all {B} pools and every layer's selections byte-equal to the oracle's")
    nblk = (n + BLOCK - 1) // BLOCK
    s0 = torch.zeros((B, int(nblk.max())), dtype=torch.float32, device="cuda")
    csa2.block_scores(g, qt[0], s0)
    s0 = s0.cpu().numpy()
    sel1 = idxs[1].cpu().numpy()
    pool_t = pool.clone()
    s1 = torch.zeros((B, P), dtype=torch.float32, device="cuda")
    csa2.block_scores(g, qt[1], s1, cand=pool_t)
    s1 = s1.cpu().numpy()
    for b in range(B):
        nb = int(nblk[b])
        assert _sha(s0[b][:nb]) == str(gold["scan_sha"][b]), f"sequence {b}: full-scan scores differ"
        assert _sha(s1[b]) == str(gold["pool_sha"][b]), f"sequence {b}: pool scores differ"
        assert _top_keys_ok(np.arange(nb), s0[b][:nb], p[b]), b
        assert _top_keys_ok(p[b], s1[b], sel1[b]), b
    assert np.array_equal(idxs[2].cpu().numpy(), sel1)
    log(f"all {B} sequences: every scan and pool score bit-equal to the oracle's")

    rng = np.random.default_rng(44)
    picks = sorted({int(np.argmin(lengths)), int(np.argmax(lengths))} | set(rng.choice(B, 2, replace=False).tolist()))
    for b in picks:
        n0, nb = int(lengths[b]), int(nblk[b])
        qbar0 = collapse_query(qs[0][b])
        blocks = np.unique(np.concatenate([rng.choice(min(nb - 1, W.CHUNK // BLOCK), 6, replace=False), [nb - 1]]))
        want = []
        for beta in blocks.tolist():
            cnt = min(BLOCK, int(n[b]) - BLOCK * beta)
            c, s = quantize_rows(_seq_rows(w.wid, 0, b, np.arange(BLOCK * beta, BLOCK * beta + cnt), n0, step_rows[b]))
            want.append(block_scores_from_keys(qbar0, block_keys(c, s, cnt))[0])
        assert np.array_equal(s0[b][blocks].view(np.uint32), np.asarray(want, dtype=np.float32).view(np.uint32)), b
        # the Reindex layer's pool rescoring, sampled on pool blocks of the first chunk
        qbar1 = collapse_query(qs[1][b])
        near = np.flatnonzero(p[b] < W.CHUNK // BLOCK)
        pick = rng.choice(near, min(4, near.size), replace=False)
        want = []
        for beta in p[b][pick].tolist():
            cnt = min(BLOCK, int(n[b]) - BLOCK * beta)
            c, s = quantize_rows(_seq_rows(w.wid, 0, b, np.arange(BLOCK * beta, BLOCK * beta + cnt), n0, step_rows[b]))
            want.append(block_scores_from_keys(qbar1, block_keys(c, s, cnt))[0])
        assert np.array_equal(s1[b][pick].view(np.uint32), np.asarray(want, dtype=np.float32).view(np.uint32)), b
        for l in (0, 1):
            idx = idxs[l].cpu().numpy()[b]
            pos = gather_positions(idx, int(n[b]))
            codes, scales = quantize_rows(_seq_rows(w.wid, 0, b, pos, n0, step_rows[b]))
            kept = idx[idx >= 0]
            ccodes = np.zeros((BLOCK * kept.size, 256), dtype=np.uint8)
            cscales = np.zeros((BLOCK * kept.size, 32), dtype=np.uint8)
            ccodes[:pos.size] = codes
            cscales[:pos.size] = scales
            ref = sparse_attend(ccodes, cscales, pos.size, qs[l][b], np.arange(kept.size), w.scale)
            err = normwise_err(outs[l].cpu().numpy()[b][None], ref[None])
            assert err <= ATT_TOL, (b, l, err)
        log(f"sequence {b} ({n0} positions): sampled scores bit-exact, attention within {ATT_TOL}")


def test_prefill_attend_1m_4096_queries_sampled():
    """Prefill-side attention in the configuration bench.py --prefill 4096
    times: 4,096 queries at the last positions of a 1,048,576-position cache
    (GPU-quantised), 64 heads, 256 blocks per query (its own block and 255
    seeded-random earlier ones), one workgroup per query normalising its
    output in-kernel.  Every output finite; twelve sampled queries (the first
    and last two, the rest spread) against the oracle's float64 attention
    over their selected positions (rows regenerated and quantised by the
    oracle), within the 2e-3 normwise bound."""
    require_gpu()
    import dataclasses
    from oracle.prefill import prefill_attend
    _CHUNKS.clear()
    w = dataclasses.replace(W.WORKLOADS[3], pattern=(0,))          # one cache
    n = int(w.context)
    T, H, K = 4096, w.heads, w.topk
    log(f"prefill 1M: building the {n}-position cache")
    cache = bench.build_caches(w, np.array([n]), (n + 7) // 8 * 8)[0]
    cache.max_len = n
    rng = np.random.default_rng(4096)
    qpos = np.arange(n - T, n, dtype=np.int64)
    idx = np.full((T, K), -1, dtype=np.int32)
    for t, p in enumerate(qpos.tolist()):
        own = p // 8
        idx[t] = np.sort(np.concatenate([rng.choice(own, K - 1, replace=False), [own]]))
    q = W.queries(w.wid, 100, 0, T, H)
    out = torch.full((T, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    ws = csa2.prefill_workspace(T, H, K)
    csa2.prefill_attend(cache, 0, torch.from_numpy(q).cuda(), torch.from_numpy(qpos).cuda(),
                        torch.from_numpy(idx).cuda(), w.scale, out, ws)
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    sample = np.unique(np.concatenate([[0, 1, T - 2, T - 1],
                                       np.random.default_rng(5).choice(np.arange(2, T - 2), 8, replace=False)]))
    pos = np.unique((8 * idx[sample].astype(np.int64)[:, :, None] + np.arange(8)).ravel())
    pos = pos[pos < n]
    log(f"prefill 1M: oracle rows for {sample.size} queries ({pos.size} positions)")
    codes = np.zeros((n, 256), dtype=np.uint8)
    scales = np.zeros((n, 32), dtype=np.uint8)
    codes[pos], scales[pos] = quantize_rows(_rows(w.wid, 0, pos, -1, None))
    ref = prefill_attend(codes, scales, qpos[sample], q[sample], idx[sample], w.scale)
    err = normwise_err(got[sample], ref)
    log(f"prefill 1M: sampled normwise error {err:.2e}")
    assert err <= ATT_TOL
    _CHUNKS.clear()
