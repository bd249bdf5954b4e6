"""Indexer of the CSA2 global KV (oracle; test infrastructure only).

The pages say what the indexer is for, not how it scores: CSA2 looks only at
a small, most relevant subset of history positions chosen by top-k [P2 "same
notes, many layers"]; the hierarchical indexer works on blocks of 8
positions [P2, same section: 2,048 blocks x 8 = 16,384 candidates].

Readings taken (the pages are silent on every step below):
  * Block b covers positions 8b..8b+7; a partial last block holds
    cnt = n - 8b < 8 positions and is scored like the others.
  * Block key K_b[c] = mean of the block's dequantised rows: the rows are
    added in ascending position order in float32, then divided by cnt in
    float32 (IEEE, correctly rounded).  With cnt = 8 this is the exact x1/8.
  * Heads are collapsed into one indexer query before scoring:
    Qbar = q_0, then Qbar = fl32(Qbar + q_h) for h = 1..H-1, channel-wise.
  * Score s_b = Qbar . K_b in a pinned float32 order, because the selected
    indices must be reproducible bit for bit:
      p_c = fl32(Qbar_c * K_b[c])                 (no fused multiply-add)
      g_j = p_{16j} + p_{16j+1} + ... + p_{16j+15}   left to right, j = 0..31
            (the 16 channels that share one E4M3 scale)
      the 32 group sums are then added pairwise as a tree of adjacent pairs:
      level 1 forms g_0+g_1, g_2+g_3, ...; level 2 adds adjacent results of
      level 1; five levels in all.
      s_b = (tree result) + 0.0, which turns -0 into +0.
    No 1/sqrt(512) factor: it does not change the ranking.

Per-head variant (score = SCORE_HEADMAX).  The pages do not say how the
indexer turns many query heads into one block score.  The reading above sums
the heads first; the other plain reading scores every head on its own and
keeps the best head's score:
      s_b = max over h of S_h,b,  S_h,b = the pinned-order score above with
      q_h in place of Qbar
(the maximum is exact).  It costs one 512-term dot product per head and
block, heads times the collapsed scan's arithmetic; the pages put the whole
decode step's FLOPs at roughly a quarter more for a 256x longer context [P2
"why it matters"], which leaves room for indexer arithmetic that grows with
the context.
"""
import numpy as np

from .quantize import D, GROUP, NGROUPS, dequantize_rows

BLOCK = 8   # positions per block
SCORE_SUM, SCORE_HEADMAX = 0, 1   # heads summed into Qbar / best per-head score


def num_blocks(n: int) -> int:
    return (int(n) + BLOCK - 1) // BLOCK


def block_keys(codes, scales, n, chunk_blocks=8192):
    """Block keys of one sequence's first n positions -> float32 [nblk, 512].

    Works through the blocks in chunks only to bound memory; every block is
    reduced on its own with the same float32 steps.
    """
    n = int(n)
    nblk = num_blocks(n)
    keys = np.empty((nblk, D), dtype=np.float32)
    for b0 in range(0, nblk, chunk_blocks):
        b1 = min(nblk, b0 + chunk_blocks)
        p0, p1 = BLOCK * b0, min(n, BLOCK * b1)
        rows = dequantize_rows(codes[p0:p1], scales[p0:p1])   # exact float32
        nfull = (p1 - p0) // BLOCK
        full = rows[:nfull * BLOCK].reshape(nfull, BLOCK, D)
        acc = full[:, 0].copy()
        for t in range(1, BLOCK):
            acc = acc + full[:, t]                         # float32 adds, t ascending
        keys[b0:b0 + nfull] = acc / np.float32(BLOCK)
        rest = (p1 - p0) - nfull * BLOCK                   # partial last block
        if rest:
            tail = rows[nfull * BLOCK:]
            acc = tail[0].copy()
            for t in range(1, rest):
                acc = acc + tail[t]
            keys[b0 + nfull] = acc / np.float32(rest)
    return keys


def collapse_query(q):
    """q float32 [H, 512] -> Qbar float32 [512], heads added in order."""
    q = np.asarray(q, dtype=np.float32)
    if not np.all(np.isfinite(q)):
        raise ValueError("non-finite query")
    acc = q[0].copy()
    for h in range(1, q.shape[0]):
        acc = acc + q[h]
    return acc


def pinned_dot(qbar, key):
    """Score of one block key against Qbar in the pinned float32 order."""
    qbar = np.asarray(qbar, dtype=np.float32)
    key = np.asarray(key, dtype=np.float32)
    p = qbar * key                                        # float32 products
    groups = []
    for j in range(NGROUPS):
        acc = p[GROUP * j]
        for c in range(GROUP * j + 1, GROUP * (j + 1)):
            acc = np.float32(acc + p[c])
        groups.append(acc)
    level = groups
    while len(level) > 1:
        level = [np.float32(level[i] + level[i + 1]) for i in range(0, len(level), 2)]
    return np.float32(level[0] + np.float32(0.0))


def block_scores_from_keys(qbar, keys):
    """Pinned-order scores of many keys at once -> float32 [nblk].

    The same arithmetic as ``pinned_dot``, run across blocks with NumPy
    float32 arrays: each step is one IEEE operation per block.
    """
    qbar = np.asarray(qbar, dtype=np.float32)
    keys = np.asarray(keys, dtype=np.float32)
    p = keys * qbar[None, :]
    p = p.reshape(keys.shape[0], NGROUPS, GROUP)
    acc = p[:, :, 0].copy()
    for c in range(1, GROUP):
        acc = acc + p[:, :, c]
    while acc.shape[1] > 1:
        acc = acc[:, 0::2] + acc[:, 1::2]
    return acc[:, 0] + np.float32(0.0)


def headmax_scores_from_keys(q, keys):
    """Per-head variant: for every key, the largest over the heads q [H, 512]
    of that head's pinned-order score (block_scores_from_keys with q_h in
    place of Qbar) -> float32 [nblk]."""
    q = np.asarray(q, dtype=np.float32)
    if not np.all(np.isfinite(q)):
        raise ValueError("non-finite query")
    best = block_scores_from_keys(q[0], keys)
    for h in range(1, q.shape[0]):
        best = np.maximum(best, block_scores_from_keys(q[h], keys))
    return best


def block_scores(codes, scales, n, q, cand=None, score=SCORE_SUM):
    """Scores of one sequence's blocks for the query heads q [H, 512].

    cand: block ids to score (None = all blocks).  score: SCORE_SUM (heads
    summed into Qbar) or SCORE_HEADMAX (best per-head score).
    Returns (ids, scores).
    """
    keys = block_keys(codes, scales, n)
    ids = np.arange(keys.shape[0], dtype=np.int64) if cand is None else \
        np.asarray([c for c in cand if c >= 0], dtype=np.int64)
    if ids.size and (ids.max() >= keys.shape[0]):
        raise ValueError("candidate block id out of range")
    if score == SCORE_HEADMAX:
        return ids, headmax_scores_from_keys(q, keys[ids])
    if score != SCORE_SUM:
        raise ValueError(f"unknown score rule {score}")
    qbar = collapse_query(q)
    return ids, block_scores_from_keys(qbar, keys[ids])
