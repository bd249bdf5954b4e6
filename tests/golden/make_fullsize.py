#!/usr/bin/env python3
"""Write the full-size expected values of the GPU parity tests.

Every value written here comes from the CPU oracle (``oracle/``) run on the
seeded synthetic inputs of ``workloads/``; nothing is read from the GPU
library.  The oracle is run on exactly the inputs the GPU tests feed the
library: the same prefill rows, appended rows and queries.

Outputs (in this directory):

  fullsize_decoder20_1m.npz   the 20-layer decoder at 1,048,576 positions
      (batch 1, 64 heads, pool 2,048, top-256, pattern [F,Ri,Ru,Ru,Ri] x 4),
      decode step 0 (one row appended to each of the 4 Full caches):
        pool        int32 [2048]   the first Full layer's candidate pool
        idx         int32 [20, 256] every layer's selection
        scan_sha    sha256 of the first layer's float32 scores of all
                    131,073 blocks (block order, little-endian bytes)
        pool_sha    sha256 of each selecting layer's float32 scores of the
                    pool blocks in pool order ("" for the first and Reuse
                    layers)
  fullsize_ragged_b64.npz     the batch workload (64 sequences of seeded
      lengths in [32,768, 131,072], [F, Ri, Ru], 16 heads, pool 2,048,
      top-128), decode step 0:
        lengths     int64 [64] prefill lengths
        pool        int32 [64, 2048]
        idx         int32 [3, 64, 128]
        scan_sha    per sequence: sha256 of its full-scan float32 scores
        pool_sha    per sequence: sha256 of the Reindex layer's pool scores
  fullsize_decoder20_1m_headmax.npz   the same step with the per-head score
      rule (score = the best head's pinned-order score): the same fields,
      the scores being per-head ones
  prefill_write_1m.json       the prefill write (1,048,576 rows of workload
      4, cache stream 9): sha256 of the oracle's codes bytes then scales
      bytes of every 65,536-row chunk.

Run from the repository root (takes several minutes on 8 cores):
    python tests/golden/make_fullsize.py [decoder20|decoder20-headmax|ragged|prefill|all]
"""
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402
from oracle.indexer import (SCORE_HEADMAX, SCORE_SUM, block_keys, block_scores_from_keys,  # noqa: E402
                            collapse_query, headmax_scores_from_keys)
from oracle.quantize import quantize_rows  # noqa: E402
from oracle.step import Cache, decode_step  # noqa: E402

WORKERS = min(8, os.cpu_count() or 1)


def log(msg):
    print(f"[golden] {msg}", flush=True)


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def _quantized_chunk(job):
    wid, cache, seq, chunk, count = job
    rows = W.kv_rows(wid, cache, seq, chunk * W.CHUNK, count)
    return job, quantize_rows(rows)


def fill_cache(wid, cache_id, lengths, capacity):
    """An oracle Cache holding each sequence's prefill rows, quantised by the
    oracle (chunks in parallel processes; each chunk has its own seed)."""
    oc = Cache(len(lengths), capacity)
    jobs = []
    for b, n in enumerate(lengths):
        for k in range((int(n) + W.CHUNK - 1) // W.CHUNK):
            jobs.append((wid, cache_id, b, k, min(W.CHUNK, int(n) - k * W.CHUNK)))
    with ProcessPoolExecutor(max_workers=WORKERS) as ex:
        for (_, _, b, k, cnt), (codes, scales) in ex.map(_quantized_chunk, jobs):
            oc.codes[b, k * W.CHUNK:k * W.CHUNK + cnt] = codes
            oc.scales[b, k * W.CHUNK:k * W.CHUNK + cnt] = scales
    oc.seq_len[:] = np.asarray(lengths, dtype=np.int64)
    return oc


def _scores(q, keys, score):
    """The indexer's scores of `keys` for the query heads q [H, 512] under the rule."""
    if score == SCORE_HEADMAX:
        return headmax_scores_from_keys(q, keys)
    return block_scores_from_keys(collapse_query(q), keys)


def decoder20(score=SCORE_SUM):
    w = W.WORKLOADS[3]
    n0 = int(w.context)
    cap = (n0 + 1 + 7) // 8 * 8
    t0 = time.perf_counter()
    caches = []
    for c in range(w.n_caches):
        caches.append(fill_cache(w.wid, c, [n0], cap))
        log(f"decoder20: cache {c} quantised ({time.perf_counter() - t0:.0f} s)")
    L, H = len(w.pattern), w.heads
    lc = w.layer_caches()
    qs = [W.queries(w.wid, l, 0, 1, H) for l in range(L)]
    rows = np.stack([W.append_rows(w.wid, c, 0, 1) for c in range(w.n_caches)])
    layers = [(m, lc[l], qs[l]) for l, m in enumerate(w.pattern)]
    res = decode_step(caches, layers, rows, w.topk, w.pool, w.scale, score=score)
    log(f"decoder20: decode step done ({time.perf_counter() - t0:.0f} s)")
    n = n0 + 1
    pool = res["pool"][0]
    keys = {}
    for c in sorted(set(lc)):
        keys[c] = block_keys(caches[c].codes[0], caches[c].scales[0], n)
    scan = _scores(qs[0][0], keys[lc[0]], score)
    pool_sha = []
    for l, m in enumerate(w.pattern):
        if l == 0 or m == 2:
            pool_sha.append("")
            continue
        pool_sha.append(sha(_scores(qs[l][0], keys[lc[l]][pool], score)))
    name = "fullsize_decoder20_1m_headmax.npz" if score == SCORE_HEADMAX else "fullsize_decoder20_1m.npz"
    np.savez_compressed(os.path.join(HERE, name),
                        pool=pool.astype(np.int32), idx=np.stack([i[0] for i in res["idx"]]).astype(np.int32),
                        scan_sha=np.array(sha(scan)), pool_sha=np.array(pool_sha))
    log(f"decoder20: written ({time.perf_counter() - t0:.0f} s)")


def ragged():
    w = W.WORKLOADS[4]
    lengths = W.lengths(w)
    B = len(lengths)
    cap = int((int(lengths.max()) + 1 + 7) // 8 * 8)
    t0 = time.perf_counter()
    cache = fill_cache(w.wid, 0, lengths, cap)
    log(f"ragged: cache quantised ({time.perf_counter() - t0:.0f} s)")
    L, H = len(w.pattern), w.heads
    qs = [W.queries(w.wid, l, 0, B, H) for l in range(L)]
    rows = W.append_rows(w.wid, 0, 0, B)[None]
    layers = [(m, 0, qs[l]) for l, m in enumerate(w.pattern)]
    res = decode_step([cache], layers, rows, w.topk, w.pool, w.scale)
    log(f"ragged: decode step done ({time.perf_counter() - t0:.0f} s)")
    pool = res["pool"]
    scan_sha, pool_sha = [], []
    for b in range(B):
        n = int(cache.seq_len[b])
        keys = block_keys(cache.codes[b], cache.scales[b], n)
        scan_sha.append(sha(block_scores_from_keys(collapse_query(qs[0][b]), keys)))
        pool_sha.append(sha(block_scores_from_keys(collapse_query(qs[1][b]), keys[pool[b]])))
    np.savez_compressed(os.path.join(HERE, "fullsize_ragged_b64.npz"),
                        lengths=lengths.astype(np.int64), pool=pool.astype(np.int32),
                        idx=np.stack(res["idx"]).astype(np.int32),
                        scan_sha=np.array(scan_sha), pool_sha=np.array(pool_sha))
    log(f"ragged: written ({time.perf_counter() - t0:.0f} s)")


def _prefill_chunk(k):
    rows = W.kv_rows(4, 9, 0, k * W.CHUNK, W.CHUNK)
    codes, scales = quantize_rows(rows)
    return k, sha(codes), sha(scales)


def prefill():
    R = 64 * W.PREFILL_WRITE_ROWS
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=WORKERS) as ex:
        got = sorted(ex.map(_prefill_chunk, range(R // W.CHUNK)))
    out = {"rows": R, "chunk_rows": W.CHUNK, "workload": 4, "cache_stream": 9,
           "codes_sha256": [g[1] for g in got], "scales_sha256": [g[2] for g in got]}
    with open(os.path.join(HERE, "prefill_write_1m.json"), "w") as f:
        json.dump(out, f, indent=1)
    log(f"prefill: written ({time.perf_counter() - t0:.0f} s)")


if __name__ == "__main__":
    what = sys.argv[1] if len(sys.argv) > 1 else "all"
    if what in ("prefill", "all"):
        prefill()
    if what in ("decoder20", "all"):
        decoder20()
    if what in ("decoder20-headmax", "all"):
        decoder20(SCORE_HEADMAX)
    if what in ("ragged", "all"):
        ragged()
