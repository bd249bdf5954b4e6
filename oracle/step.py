"""Layer-stack driver for one decode step (oracle; test infrastructure only).

CSA2 gives every decoder layer one fixed mode [P2 "same notes, many layers";
P3 section 二, mode table]:
  Full     the layer writes its own global KV and selects its own top-k;
  Reindex  the layer reuses the earlier layer's KV but selects again;
  Reuse    the layer reuses both the KV and the earlier layer's selection,
           computing neither.
Hierarchical sparse indexer [P2, same section]: the decoder's first Full
layer scans the whole range and keeps a larger candidate pool (2,048 blocks
of 8 positions in the page's example); later layers search only that pool,
so their cost stops growing with the context, while the first scan remains.

Readings (the pages leave these open):
  * "the earlier layer's KV" is the cache of the most recent Full layer;
    "the earlier layer's selection" is the selection of the layer just before
    (for a Reuse chain this is, transitively, the last selecting layer).
  * Every selecting layer after the first Full layer searches the pool,
    a later Full layer on its own cache, a Reindex layer on the latest Full
    cache.  The first Full layer attends to its own top-k, which lies inside
    its pool.  With pool size 0 every selecting layer scans all blocks.
  * Step order: each Full cache first appends this step's new row for every
    sequence (quantised like every other row), then the layers run in order.
  * Optional local branch (oracle/swa.py): a layer with an SWA cache writes
    its own FP8 row for the new token and attends to its window together
    with its CSA2 positions in one softmax.
"""
import numpy as np

from . import attend as _attend
from . import indexer as _indexer
from . import swa as _swa
from .quantize import BYTES_PER_TOKEN, CODE_BYTES, D, SCALE_BYTES, quantize_rows
from .select import select

FULL, REINDEX, REUSE = 0, 1, 2


class Cache:
    """One Full layer's FP4 cache for a batch of sequences."""

    def __init__(self, batch, capacity):
        if capacity % _indexer.BLOCK:
            raise ValueError("capacity must be a multiple of 8")
        self.codes = np.zeros((batch, capacity, CODE_BYTES), dtype=np.uint8)
        self.scales = np.zeros((batch, capacity, SCALE_BYTES), dtype=np.uint8)
        self.seq_len = np.zeros(batch, dtype=np.int64)

    @property
    def batch(self):
        return self.codes.shape[0]

    @property
    def capacity(self):
        return self.codes.shape[1]

    def write(self, b, start, rows):
        """Quantise float32 rows [m, 512] into positions start.. of sequence b."""
        rows = np.asarray(rows, dtype=np.float32).reshape(-1, D)
        if start + rows.shape[0] > self.capacity:
            raise ValueError("cache capacity exceeded")
        c, s = quantize_rows(rows)
        self.codes[b, start:start + rows.shape[0]] = c
        self.scales[b, start:start + rows.shape[0]] = s

    def append(self, rows):
        """Append one row per sequence (float32 [B, 512]); seq_len += 1."""
        rows = np.asarray(rows, dtype=np.float32).reshape(self.batch, D)
        for b in range(self.batch):
            self.write(b, int(self.seq_len[b]), rows[b:b + 1])
            self.seq_len[b] += 1


def decode_step(caches, layers, new_rows, topk, pool, scale, swa=None, swa_rows=None, window=0,
                score=_indexer.SCORE_SUM):
    """Run one decode step.

    caches:   list of Cache (one per Full layer); mutated by the append.
    layers:   list of (mode, cache_index, q float32 [B, H, 512]).
    new_rows: float32 [n_caches, B, 512] appended first, or None.
    swa:      None, or one swa.SwaCache (or None) per layer: the layer's local
              branch, window positions wide; swa_rows float32 [n_layers, B, 512]
              (rows of layers without a cache are ignored) are appended first.
    score:    the indexer's head rule, SCORE_SUM (heads summed) or
              SCORE_HEADMAX (best per-head score) (oracle/indexer.py).
    Returns dict with 'idx' (list of int32 [B, topk]), 'out' (list of float64
    [B, H, 512]) and 'pool' (int32 [B, pool] or None).
    """
    if new_rows is not None:
        for ci, cache in enumerate(caches):
            cache.append(new_rows[ci])
    B = caches[0].batch
    pool_ids = None
    prev_idx = None
    latest_full = None
    idx_all, out_all = [], []
    for li, (mode, ci, q) in enumerate(layers):
        q = np.asarray(q, dtype=np.float32)
        if mode == FULL:
            latest_full = ci
        else:
            if latest_full is None:
                raise ValueError(f"layer {li}: no earlier Full layer")
            if ci != latest_full:
                raise ValueError(f"layer {li}: must use the latest Full cache")
        cache = caches[ci]
        if mode == REUSE:
            if prev_idx is None:
                raise ValueError(f"layer {li}: Reuse with no earlier selection")
            idx = prev_idx.copy()
        else:
            idx = np.full((B, topk), -1, dtype=np.int32)
            build_pool = pool > 0 and pool_ids is None
            if build_pool:
                pool_ids = np.full((B, pool), -1, dtype=np.int32)
            for b in range(B):
                n = int(cache.seq_len[b])
                if pool > 0 and not build_pool:
                    cand = pool_ids[b]
                else:
                    cand = None
                ids, sc = _indexer.block_scores(cache.codes[b], cache.scales[b], n, q[b], cand, score)
                if build_pool:
                    pool_ids[b] = select(ids, sc, pool)
                    keep = np.isin(ids, pool_ids[b])
                    ids, sc = ids[keep], sc[keep]
                idx[b] = select(ids, sc, topk)
        sw = swa[li] if swa is not None else None
        if sw is not None:
            sw.append(swa_rows[li])
            out = np.stack([
                _swa.attend_with_window(cache.codes[b], cache.scales[b], int(cache.seq_len[b]),
                                        q[b], idx[b], scale, sw.codes[b], sw.scales[b],
                                        int(sw.seq_len[b]), window)
                for b in range(B)])
        else:
            out = np.stack([
                _attend.sparse_attend(cache.codes[b], cache.scales[b], int(cache.seq_len[b]),
                                      q[b], idx[b], scale)
                for b in range(B)])
        idx_all.append(idx)
        out_all.append(out)
        prev_idx = idx
    return {"idx": idx_all, "out": out_all, "pool": pool_ids}


__all__ = ["Cache", "decode_step", "FULL", "REINDEX", "REUSE", "BYTES_PER_TOKEN"]
