"""Seeded synthetic workloads for the CSA2 FP4 decode path.

Shared by the tests, the smoke check and the benchmark; it holds none of the
method's arithmetic (no quantisation, scoring, selection or attention): it
only makes float32 inputs and states the workload shapes.

Value recipe.  After rotation and normalisation KV values are close to
normal with few outliers [P1 section 二]; RMSNorm weights are at most about 1
and a norm-preserving rotation keeps the 512-channel latent's L2 norm at
most sqrt(512) ~ 22.6 [P3 section 三].  So a KV row is
    N(0,1) float32 draw -> RMSNorm (weight 1, eps 1e-6) -> one fixed random
    orthogonal 512x512 rotation per workload (Haar: QR of a Gaussian matrix
    with the signs of R's diagonal folded into Q),
and its float32 values are the shared input of both sides.  Queries are
float32 N(0,1), a fresh draw per layer and step.  Ragged lengths are uniform
integers in [32768, 131072].

Every draw comes from NumPy's PCG64 seeded by SeedSequence([workload, stream,
...]); KV rows are drawn in chunks of 65,536 positions so that any position
can be regenerated on its own.
"""
from dataclasses import dataclass, field

import numpy as np

D = 512
CHUNK = 65536

STREAM_KV, STREAM_ROT, STREAM_Q, STREAM_APPEND, STREAM_LEN = 1, 2, 3, 4, 5
STREAM_SWA, STREAM_SWA_APPEND = 6, 7

FULL, REINDEX, REUSE = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    batch: int
    context: int                 # prefilled positions (ragged: see lengths())
    heads: int
    topk: int
    pool: int
    pattern: tuple               # mode per layer
    steps: int                   # decode steps per run
    append: bool                 # whether each step appends one row per Full cache
    ragged: tuple = None         # (lo, hi) inclusive, or None
    scale: float = 1.0 / np.sqrt(512.0)
    note: str = field(default="", compare=False)

    @property
    def n_caches(self):
        return sum(1 for m in self.pattern if m == FULL)

    def layer_caches(self):
        """Cache index of each layer: Full layers own caches in order; the
        others use the latest Full cache."""
        out, cur = [], -1
        for m in self.pattern:
            if m == FULL:
                cur += 1
            out.append(cur)
        return out


WORKLOADS = {
    0: Workload(0, "single-full-4k", 1, 4096, 16, 64, 0, (FULL,), 1, False,
                note="one Full layer, batch 1, 4,096 positions, 16 heads, top-64"),
    1: Workload(1, "full-reindex-reuse-64k-b4", 4, 65536, 16, 256, 0,
                (FULL, REINDEX, REUSE), 1, False,
                note="Full->Reindex->Reuse, batch 4, 65,536 positions, no pool"),
    2: Workload(2, "hier-pool-256k", 1, 262144, 64, 256, 2048,
                (FULL, REINDEX, REINDEX), 1, False,
                note="Full scan into a 2,048-block pool, then two pool-only Reindex layers"),
    3: Workload(3, "decoder20-1m", 1, 1 << 20, 64, 256, 2048,
                (FULL, REINDEX, REUSE, REUSE, REINDEX) * 4, 50, True,
                note="20 layers [F,Ri,Ru,Ru,Ri]x4 at 1,048,576 positions, 50 appending steps"),
    4: Workload(4, "ragged-b64", 64, 0, 16, 128, 2048, (FULL, REINDEX, REUSE), 50, True,
                ragged=(32768, 131072),
                note="batch 64, ragged 32K-128K, Full/Reindex/Reuse, 50 appending steps"),
}

PREFILL_WRITE_ROWS = 16384   # per sequence, batch 64: the quantiser throughput test


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


_ROT_CACHE = {}


def rotation(wid):
    """Haar-random orthogonal 512x512 (float64) for one workload."""
    if wid not in _ROT_CACHE:
        g = _rng(wid, STREAM_ROT).standard_normal((D, D))
        qm, r = np.linalg.qr(g)
        qm = qm * np.sign(np.diag(r))[None, :]
        _ROT_CACHE[wid] = qm
    return _ROT_CACHE[wid]


def shape_rows(z, wid):
    """RMSNorm (weight 1) then the workload's rotation; float32 out.

    The rotation is applied in float64 and rounded once to float32, so the
    rows do not depend on the host's matrix-multiply kernel: a float32
    product's summation order varies with the BLAS build and CPU, a float64
    one changes the rounded float32 value only with a ~1e-9 chance per value.
    """
    z = np.asarray(z, dtype=np.float32)
    rms = np.sqrt(np.mean(z.astype(np.float64) ** 2, axis=-1, keepdims=True) + 1e-6)
    zn = (z / rms).astype(np.float32)
    return (zn.astype(np.float64) @ rotation(wid)).astype(np.float32)


def _kv_chunk(wid, cache, seq, chunk):
    z = _rng(wid, STREAM_KV, cache, seq, chunk).standard_normal((CHUNK, D), dtype=np.float32)
    return shape_rows(z, wid)


def kv_rows(wid, cache, seq, start, count):
    """Prefill rows [start, start+count) of (cache, sequence) -> float32 [count, 512]."""
    out = np.empty((count, D), dtype=np.float32)
    p = start
    while p < start + count:
        c = p // CHUNK
        lo = p - c * CHUNK
        hi = min(CHUNK, start + count - c * CHUNK)
        out[p - start:p - start + hi - lo] = _kv_chunk(wid, cache, seq, c)[lo:hi]
        p += hi - lo
    return out


def kv_chunks(wid, cache, seq, count):
    """Yield (start, rows) chunks covering positions [0, count)."""
    for c in range((count + CHUNK - 1) // CHUNK):
        rows = _kv_chunk(wid, cache, seq, c)
        n = min(CHUNK, count - c * CHUNK)
        yield c * CHUNK, rows[:n]


def kv_rows_threaded(wid, cache, seq, count, threads=8):
    """kv_rows(wid, cache, seq, 0, count), chunks drawn on a thread pool
    (each chunk has its own seed, so the result does not depend on threads)."""
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty((count, D), dtype=np.float32)
    nchunk = (count + CHUNK - 1) // CHUNK

    def one(c):
        n = min(CHUNK, count - c * CHUNK)
        out[c * CHUNK:c * CHUNK + n] = _kv_chunk(wid, cache, seq, c)[:n]

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(nchunk)))
    return out


def queries(wid, layer, step, batch, heads):
    """Query heads of one layer at one step -> float32 [B, H, 512]."""
    return _rng(wid, STREAM_Q, layer, step).standard_normal((batch, heads, D), dtype=np.float32)


def append_rows(wid, cache, step, batch):
    """Rows appended by one Full cache at one step -> float32 [B, 512]."""
    z = _rng(wid, STREAM_APPEND, cache, step).standard_normal((batch, D), dtype=np.float32)
    return shape_rows(z, wid)


def swa_rows(wid, layer, seq, start, count):
    """Sliding-window (local branch) rows of one layer, positions
    [start, start+count) of one sequence -> float32 [count, 512]; shaped like
    the global rows (RMSNorm, rotation)."""
    z = _rng(wid, STREAM_SWA, layer, seq, start).standard_normal((count, D), dtype=np.float32)
    return shape_rows(z, wid)


def swa_append_rows(wid, layer, step, batch):
    """Local-branch rows one layer writes at one decode step -> float32 [B, 512]."""
    z = _rng(wid, STREAM_SWA_APPEND, layer, step).standard_normal((batch, D), dtype=np.float32)
    return shape_rows(z, wid)


def lengths(w: Workload):
    """Prefilled length of each sequence -> int64 [B]."""
    if w.ragged is None:
        return np.full(w.batch, w.context, dtype=np.int64)
    lo, hi = w.ragged
    return _rng(w.wid, STREAM_LEN).integers(lo, hi, size=w.batch, endpoint=True).astype(np.int64)


def scaled(w: Workload, context=None, batch=None, steps=None, pool=None, topk=None, heads=None):
    """A smaller copy of a workload (same pattern and recipe) for quick tests."""
    kw = dict(w.__dict__)
    for k, v in (("context", context), ("batch", batch), ("steps", steps),
                 ("pool", pool), ("topk", topk), ("heads", heads)):
        if v is not None:
            kw[k] = v
    if context is not None:
        kw["ragged"] = None
    return Workload(**kw)
