"""Helpers of the GPU parity tests: oracle-built caches uploaded to the GPU.

Cache bytes always come from the oracle's quantiser (or the pages'
formats), never from the HIP path, so the scoring/selection/attention
parity tests compare both sides on identical inputs.
"""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
import workloads as W
from oracle.step import Cache


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.load()   # raises if the HIP library is missing: no fallback


def oracle_cache(wid, cache_id, lengths, capacity):
    """An oracle Cache whose sequences hold workload rows quantised by the oracle."""
    lengths = [int(n) for n in lengths]
    c = Cache(len(lengths), capacity)
    for b, n in enumerate(lengths):
        for start, rows in W.kv_chunks(wid, cache_id, b, n):
            c.write(b, start, rows)
        c.seq_len[b] = n
    return c


def to_device(oc, max_len=None):
    B, cap = oc.codes.shape[:2]
    g = csa2.KVCache(B, cap)
    g.codes.copy_(torch.from_numpy(oc.codes))
    g.scales.copy_(torch.from_numpy(oc.scales))
    g.seq_len.copy_(torch.from_numpy(oc.seq_len))
    g.max_len = int(oc.seq_len.max()) if max_len is None else max_len
    return g


def normwise_err(out, ref):
    """max over rows of ||out - ref||_inf / ||ref||_inf (rows with ref == 0: absolute)."""
    out = np.asarray(out, dtype=np.float64).reshape(-1, out.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    num = np.abs(out - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1), num)))


ATT_TOL = 2e-3   # max relative error of the attention outputs (normwise per row)


def cap_for(n, extra=0):
    return int((n + extra + 7) // 8 * 8) or 8


def log(msg):
    print(msg, flush=True)
