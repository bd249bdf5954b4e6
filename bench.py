#!/usr/bin/env python3
"""Decode-step benchmark of the CSA2 FP4 global-KV hot path on one MI355X.

One step = one decode step of the whole hot path for the 20-layer decoder
pattern [Full, Reindex, Reuse, Reuse, Reindex] x 4 at a 1,048,576-position
context (batch 1, 64 heads, pool 2,048 blocks, top-256): append one
quantised row to each of the 4 Full caches, full-range scan of the first Full
layer into the pool, top-k, pool rescoring in the 11 later selecting layers,
Reuse forwarding and sparse attention in all 20 layers.  Inputs (caches,
queries, appended rows) are synthetic and resident in HBM before timing.

Prints one JSON line (metric, value = decode tokens/s, roofline of the
dominant kernel, CPU-oracle baseline).  Progress goes to stderr.

  python bench.py [--steps K] [--warmup W] [--gpus 1]
  python bench.py --copy-probe     (plain copy kernel for counter calibration)
  python bench.py --prefill 4096   (prefill-side sparse attention, its own JSON line)
  python bench.py --prefill-write  (FP4 quantisation of 1,048,576 prompt rows, its own JSON line)
  python bench.py --cpu-only [--cpu-steps N] [--cpu-threads N]   (the oracle baseline alone)
  python bench.py --launch-floor   (a chain of dependent tiny launches: the per-launch floor)
  python bench.py --score headmax  (the per-head indexer score rule: every head scores each block
                                    in the pinned float32 order, the best head's score ranks it)

By default the 256 MB last-level cache is flushed (a 512 MB read) between
the timed steps and the step time is the mean of the events around each
step; --warm runs them back to back.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
# Vector ALU peak for float32 work that may use neither FMA nor packed math
# (the per-head score's pinned order multiplies and adds separately): 256
# compute units x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3 T operations/s, each
# multiply or add one operation (the published 157.3 TFLOP/s counts packed
# FMAs, 4 flops per lane per clock).
PEAK_VALU_TOPS = 256 * 64 * 2.4e9 / 1e12
TOKEN_BYTES = 288              # 256 code bytes + 32 scale bytes per position
BLOCK_BYTES = 8 * TOKEN_BYTES  # 2,304
PMC_FILE = os.path.join(ROOT, "profiles", "scan_kernel_decoder20-1m_pmc.txt")
PMC_FILE_FLAT = os.path.join(ROOT, "profiles", "scan_flat_kernel_ragged-b64_pmc.txt")
SCAN_SOURCES = [os.path.join(ROOT, "fp4_compressed_sparse_amd", "csrc", f)
                for f in ("index.hip", "common.hpp")]
QUANT_PMC_FILE = os.path.join(ROOT, "profiles", "quantize_rows_kernel_prefill-write-1m_pmc.txt")
QUANT_SOURCES = [os.path.join(ROOT, "fp4_compressed_sparse_amd", "csrc", f)
                 for f in ("quantize.hip", "common.hpp", "api.hip")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def scan_source_sha():
    return source_sha(SCAN_SOURCES)


def step_bytes(w, n_tokens):
    """Algorithmic KV bytes of one step: (unique, touched), per sequence
    lengths n_tokens (after the append)."""
    unique = touched = 0
    for n in n_tokens:
        nblk = (n + 7) // 8
        first = True
        pool_blocks = min(w.pool, nblk) if w.pool else 0
        full_count = 0
        for m in w.pattern:
            if m != 2:                         # selecting layer
                if first:
                    touched += n * TOKEN_BYTES
                    unique += n * TOKEN_BYTES
                    first = False
                elif w.pool:
                    touched += pool_blocks * BLOCK_BYTES
                    if m == 0:                 # a later Full layer reads its own cache's pool blocks
                        unique += pool_blocks * BLOCK_BYTES
                else:
                    touched += n * TOKEN_BYTES
                    if m == 0:
                        unique += n * TOKEN_BYTES
            if m == 0:
                full_count += 1
            touched += min(w.topk, nblk) * BLOCK_BYTES   # attention gather
    return unique, touched


def build_caches(w, lengths, capacity, log_every=8):
    """GPU caches filled with the workload's rows, quantised on the GPU."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    import fp4_compressed_sparse_amd as csa2
    import workloads as W

    caches = [csa2.KVCache(w.batch, capacity) for _ in range(w.n_caches)]
    jobs = []
    for c in range(w.n_caches):
        for b, n in enumerate(lengths):
            for k in range((int(n) + W.CHUNK - 1) // W.CHUNK):
                jobs.append((c, b, k, min(W.CHUNK, int(n) - k * W.CHUNK)))

    def gen(job):
        c, b, k, cnt = job
        return job, W._kv_chunk(w.wid, c, b, k)[:cnt]

    done = 0
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
        for (c, b, k, cnt), rows in ex.map(gen, jobs):
            x = torch.from_numpy(np.ascontiguousarray(rows)).cuda()
            s0 = k * W.CHUNK
            csa2.fp4_quantize_kv(x, caches[c].codes[b, s0:s0 + cnt], caches[c].scales[b, s0:s0 + cnt])
            done += 1
            if done % log_every == 0 or done == len(jobs):
                log(f"caches: {done}/{len(jobs)} chunks")
    for cache in caches:
        cache.seq_len.copy_(torch.as_tensor(lengths, dtype=torch.int64))
    torch.cuda.synchronize()
    return caches


def cpu_threads(threads):
    """Context that limits the host's BLAS/OpenMP pools to `threads` (0: the
    pools' own size), and the thread count in effect inside it."""
    import contextlib
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:                               # pragma: no cover
        return contextlib.nullcontext(), 1
    if threads > 0:
        return threadpool_limits(limits=threads), threads
    n = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return contextlib.nullcontext(), n


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_chunk(job):
    """One chunk of a workload cache's prefill rows, quantised by the oracle."""
    import workloads as W
    from oracle.quantize import quantize_rows
    wid, cache, seq, chunk, count = job
    return job, quantize_rows(W.kv_rows(wid, cache, seq, chunk * W.CHUNK, count))


def oracle_caches(w, lengths, capacity, workers=16):
    """The workload's Full caches holding its prefill rows quantised by the
    oracle's own quantiser (chunks in worker processes).  Call it before
    anything touches the GPU: the workers are forked from this process."""
    from concurrent.futures import ProcessPoolExecutor

    import workloads as W
    from oracle.step import Cache

    caches = [Cache(len(lengths), capacity) for _ in range(w.n_caches)]
    jobs = [(w.wid, c, b, k, min(W.CHUNK, int(n) - k * W.CHUNK))
            for c in range(w.n_caches) for b, n in enumerate(lengths)
            for k in range((int(n) + W.CHUNK - 1) // W.CHUNK)]
    with ProcessPoolExecutor(max_workers=min(workers, os.cpu_count() or 1)) as ex:
        for (_, c, b, k, cnt), (codes, scales) in ex.map(_oracle_chunk, jobs):
            caches[c].codes[b, k * W.CHUNK:k * W.CHUNK + cnt] = codes
            caches[c].scales[b, k * W.CHUNK:k * W.CHUNK + cnt] = scales
    for cache in caches:
        cache.seq_len[:] = lengths
    return caches


def cpu_baseline(w, window=0, threads=1, steps=1, score=0):
    """The oracle's decode step timed on the host at the workload's full size:
    its caches quantised by the oracle (not timed), then `steps` decode steps
    of the same layer pattern, each appending one row per Full cache as the
    GPU steps do, at `threads` host threads (0: the BLAS pool's size).
    window > 0: every layer with its local branch, as the GPU step."""
    import dataclasses

    import numpy as np

    import workloads as W
    from oracle.step import decode_step
    from oracle.swa import SwaCache

    full_batch = w.batch
    if w.batch > 4:
        # a bounded sample: the first 4 sequences (the same seeded lengths)
        w = dataclasses.replace(w, batch=4)
    lengths = W.lengths(w)
    t0 = time.perf_counter()
    caches = oracle_caches(w, lengths, int((int(lengths.max()) + steps + 7) // 8 * 8))
    log(f"cpu oracle: caches quantised by the oracle in {time.perf_counter() - t0:.1f} s")
    lc = w.layer_caches()
    L = len(w.pattern)
    swa = None
    if window:
        swa = []
        for l in range(L):
            sw = SwaCache(w.batch, int(lengths.max()) + steps)
            for b, n in enumerate(lengths):
                n = int(n)
                sw.write(b, n - window, W.swa_rows(w.wid, l, b, n - window, window))
                sw.seq_len[b] = n
            swa.append(sw)
    ctx, used = cpu_threads(threads)
    times = []
    with ctx:
        for s in range(steps):
            layers = [(m, lc[l], W.queries(w.wid, l, s, w.batch, w.heads)) for l, m in enumerate(w.pattern)]
            rows = np.stack([W.append_rows(w.wid, c, s, w.batch) for c in range(w.n_caches)]) if w.append else None
            srows = np.stack([W.swa_append_rows(w.wid, l, s, w.batch) for l in range(L)]) if window else None
            t1 = time.perf_counter()
            decode_step(caches, layers, rows, w.topk, w.pool, w.scale, swa=swa, swa_rows=srows, window=window,
                        score=score)
            times.append(time.perf_counter() - t1)
            log(f"cpu oracle: step {s}: {times[-1]:.2f} s on {used} host thread(s)")
    total = sum(times)
    return {
        "value": round(w.batch * steps / total, 6),
        "unit": "tokens/s",
        "cores": used,
        "kind": "oracle",
        "sample": (f"{steps} decode step(s) of the workload ({w.name}: batch {w.batch}"
                   + (f" of its {full_batch} sequences" if full_batch != w.batch else "") + ", "
                   f"{int(lengths.max())} positions, {L} layers, {w.heads} heads, pool {w.pool}, top-{w.topk}"
                   + (f", a {window}-position window on every layer" if window else "")
                   + (", per-head score rule" if score else "") + ") on "
                   f"{used} host thread(s) of a {cpu_model()}: " + ", ".join(f"{t:.2f}" for t in times)
                   + " s per step (caches quantised by the oracle beforehand, not timed)"),
    }


def pmc_traffic(path=PMC_FILE, sources=SCAN_SOURCES):
    """HBM bytes per launch from a committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's readings), if it
    was taken on the current kernel sources; else None.  Default: the scan."""
    try:
        with open(path) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha") != source_sha(sources):
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


class HipEvents:
    """Raw HIP events (the library records them itself, so torch's Event
    wrapper cannot be used to read them back)."""

    def __init__(self):
        import ctypes
        for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                self.hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        self.ct = ctypes

    def create(self):
        ev = self.ct.c_void_p()
        if self.hip.hipEventCreate(self.ct.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def launch_floor(args):
    """A chain of dependent tiny launches (torch's in-place add on 32K
    floats, 128 workgroups) timed with events: the per-launch floor of any
    chain of dependent kernels on this GPU."""
    import numpy as np
    import torch
    torch.cuda.set_device(0)
    x = torch.zeros(128 * 256, dtype=torch.float32, device="cuda")
    n = 40
    for _ in range(n):
        x.add_(1.0)
    torch.cuda.synchronize()
    per = []
    for _ in range(max(args.steps, 5)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            x.add_(1.0)
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) * 1e3 / n)
    print(json.dumps({"launch_floor_us_per_dependent_launch": round(float(np.median(per)), 3),
                      "chain": n, "repeats": len(per), "kernel": "torch add_ on 32,768 floats"}))


def copy_probe():
    """A plain device copy of 1 GiB (read 1 GiB, write 1 GiB), repeated: the
    reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 3}))


def read_probe(args):
    """The achievable HBM read rate for the full scan's byte count at 1M
    (301,990,608 B): csa2_read_probe (16-byte loads, the scan's 512
    workgroups) timed with events, cold (a 512 MB read before each run, as
    in the decode bench) and back to back."""
    import numpy as np
    import torch
    import fp4_compressed_sparse_amd as csa2
    torch.cuda.set_device(0)
    nbytes = 301990608 // 16 * 16
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(512 * 256, dtype=torch.int32, device="cuda")
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    flush_sink = torch.zeros((), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for mode in ("cold", "warm"):
        us = []
        for i in range(max(args.steps, 5) + 2):
            if mode == "cold":
                torch.sum(flush, dim=0, out=flush_sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            csa2.read_probe(buf, sink, stream)
            b.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                us.append(a.elapsed_time(b) * 1e3)
        med = float(np.median(us))
        res[mode] = {"median_us": round(med, 2), "tb_s": round(nbytes / med / 1e6, 3), "runs": len(us)}
    print(json.dumps({"read_probe_bytes": nbytes, "workgroups": 512, **res}))


def prefill_bench(args):
    """Batched prefill-side sparse attention (csa2_prefill_attend): T queries
    at the last T positions of one 1,048,576-position cache, each with its
    own seeded selection of 256 blocks at or before its own block."""
    import dataclasses

    import numpy as np
    import torch

    import fp4_compressed_sparse_amd as csa2
    import workloads as W

    csa2.load()
    torch.cuda.set_device(0)
    w = dataclasses.replace(W.WORKLOADS[3], pattern=(0,))          # one cache
    n = int(w.context)
    T, H, K = args.prefill, w.heads, w.topk
    t0 = time.perf_counter()
    cache = build_caches(w, np.array([n]), (n + 7) // 8 * 8)[0]
    cache.max_len = n
    log(f"cache built in {time.perf_counter() - t0:.1f} s")
    rng = np.random.default_rng(4096)
    qpos = np.arange(n - T, n, dtype=np.int64)
    idx = np.full((T, K), -1, dtype=np.int32)
    for t, p in enumerate(qpos.tolist()):
        own = p // 8
        sel = np.sort(np.concatenate([rng.choice(own, K - 1, replace=False), [own]]))
        idx[t] = sel
    positions = int(sum(min(8, int(p) + 1 - 8 * int(b)) for t, p in enumerate(qpos.tolist())
                        for b in idx[t].tolist()))
    q = torch.from_numpy(W.queries(w.wid, 100, 0, T, H)).cuda()
    qp, it = torch.from_numpy(qpos).cuda(), torch.from_numpy(idx).cuda()
    out = torch.empty((T, H, 512), dtype=torch.float32, device="cuda")
    ws = csa2.prefill_workspace(T, H, K)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        csa2.prefill_attend(cache, 0, q, qp, it, w.scale, out, ws)
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    reps = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    t_start = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        csa2.prefill_attend(cache, 0, q, qp, it, w.scale, out, ws)
        b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    launch_s = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
    flops = 4.0 * H * 512 * positions
    tflops = flops / launch_s / 1e12
    gather = positions * TOKEN_BYTES
    log(f"prefill: {T} queries, {positions} attended positions: {launch_s * 1e6:.1f} us per launch, "
        f"{tflops:.1f} TFLOP/s, gathered rows {gather / launch_s / 1e9:.0f} GB/s")
    result = {
        "metric": "prefill-side sparse attention queries/s (1M ctx, 64 heads, top-256 blocks per query, 1 GPU)",
        "value": round(T * reps / elapsed, 1),
        "unit": "queries/s",
        "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / reps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 MFMA operands, fp32 accumulate", "data": "synthetic",
        "config": {"workload": "prefill-attend-1m", "queries": T, "context": n, "heads": H,
                   "topk_blocks": K, "attended_positions": positions,
                   "median_event_launch_us": round(launch_s * 1e6, 2)},
        "roofline": {"bound": "mfma", "kernel": "attend64_kernel (all 64 heads of a query per workgroup, one split)",
                     "achieved": round(tflops, 2), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None,
                     "algorithmic_flops_per_launch": flops, "gathered_bytes_per_launch": gather},
    }
    if not args.no_cpu_baseline:
        from oracle.prefill import prefill_attend
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:                           # pragma: no cover
            threadpool_limits = None
        import contextlib
        S = 16
        rows = W.kv_rows_threaded(w.wid, 0, 0, n)      # the oracle's own copy of the cache
        from oracle.quantize import quantize_rows
        need = np.unique(np.concatenate([8 * idx[t][:, None] + np.arange(8)[None, :] for t in range(S)]).ravel())
        need = need[need < n]
        codes = np.zeros((n, 256), dtype=np.uint8)
        scales = np.zeros((n, 32), dtype=np.uint8)
        codes[need], scales[need] = quantize_rows(rows[need])
        ctx = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
        with ctx:
            t1 = time.perf_counter()
            prefill_attend(codes, scales, qpos[:S], W.queries(w.wid, 100, 0, T, H)[:S], idx[:S], w.scale)
            cpu_s = time.perf_counter() - t1
        result["cpu_baseline"] = {"value": round(S / cpu_s, 3), "unit": "queries/s", "cores": 1, "kind": "oracle",
                                  "sample": f"{S} of the {T} queries (same cache, selections and heads) on 1 host "
                                            f"thread: {cpu_s:.2f} s"}
    print(json.dumps(result), flush=True)


def prefill_write_bench(args):
    """Prefill write (fp4_quantize_kv): the batch-64 prompt's 64 x 16,384 =
    1,048,576 fresh fp32 rows, resident in HBM, quantised in one launch into
    a cache of the same size."""
    import numpy as np
    import torch

    import fp4_compressed_sparse_amd as csa2
    import workloads as W

    csa2.load()
    torch.cuda.set_device(0)
    R = 64 * W.PREFILL_WRITE_ROWS
    t0 = time.perf_counter()
    x_host = W.kv_rows_threaded(4, 9, 0, R, threads=16)
    x = torch.from_numpy(x_host).cuda()
    log(f"rows generated and copied in {time.perf_counter() - t0:.1f} s")
    codes = torch.empty((R, 256), dtype=torch.uint8, device="cuda")
    scales = torch.empty((R, 32), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        csa2.fp4_quantize_kv(x, codes, scales)
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    reps = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    t_start = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        csa2.fp4_quantize_kv(x, codes, scales)
        b.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    launch_s = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
    per_row = 512 * 4 + TOKEN_BYTES                  # fp32 row read + FP4 codes and scales written
    gbs = R * per_row / launch_s / 1e9
    log(f"prefill write: {R} rows, {launch_s * 1e6:.1f} us per launch, {gbs:.0f} GB/s")
    result = {
        "metric": "prefill write rows/s (FP4 quantisation of 1,048,576 fp32 KV rows into the cache, 1 GPU)",
        "value": round(R * reps / elapsed, 1),
        "unit": "rows/s",
        "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / reps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "prefill-write-1m", "rows": R, "sequences": 64,
                   "formats": "float32 rows in; FP4 E2M1 codes + E4M3 scales per 16 channels out",
                   "rows_per_sequence": W.PREFILL_WRITE_ROWS,
                   "median_event_launch_us": round(launch_s * 1e6, 2)},
        "roofline": {"bound": "hbm", "kernel": "quantize_rows_kernel (one lane per 16-channel group)",
                     "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs / 8000.0, 4), "traffic": pmc_traffic(QUANT_PMC_FILE, QUANT_SOURCES),
                     "algorithmic_bytes_per_launch": R * per_row},
    }
    if not args.no_cpu_baseline:
        from oracle.quantize import quantize_rows
        try:
            from threadpoolctl import threadpool_limits
        except ImportError:                           # pragma: no cover
            threadpool_limits = None
        import contextlib
        ctx = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
        C = 65536                                     # chunks bound the oracle's float64 temporaries
        with ctx:
            t1 = time.perf_counter()
            for r0 in range(0, R, C):
                quantize_rows(x_host[r0:r0 + C])
            cpu_s = time.perf_counter() - t1
        result["cpu_baseline"] = {"value": round(R / cpu_s, 1), "unit": "rows/s", "cores": 1, "kind": "oracle",
                                  "sample": f"all {R} rows, {C} at a time, on 1 host thread: {cpu_s:.2f} s"}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, help="workload id (default 3: 20 layers at 1M)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-threads", type=int, default=1, metavar="N",
                    help="host threads for the oracle baseline of the decode step (default 1; 0: the BLAS pool's size)")
    ap.add_argument("--cpu-steps", type=int, default=1, metavar="N",
                    help="oracle decode steps timed for the CPU baseline (default 1)")
    ap.add_argument("--cpu-only", action="store_true",
                    help="print only the CPU baseline of the decode step (no GPU work)")
    ap.add_argument("--launch-floor", action="store_true",
                    help="time a chain of dependent tiny launches (its own JSON line)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--read-probe", action="store_true",
                    help="achievable read rate for the 1M scan's bytes (csa2_read_probe), cold and warm")
    ap.add_argument("--prefill", type=int, default=0, metavar="T",
                    help="instead of the decode step: batched prefill-side sparse attention of T "
                         "queries (the last T positions of a 1M-position cache, 64 heads, top-256 "
                         "blocks each); prints its own JSON line")
    ap.add_argument("--prefill-write", action="store_true",
                    help="time fp4_quantize_kv over the batch-64 prompt's 1,048,576 fp32 rows (its own JSON line)")
    ap.add_argument("--swa", type=int, default=0, metavar="W",
                    help="give every layer a local branch: an FP8 sliding-window ring of W positions "
                         "(prefilled, one row appended per layer per step) attended in the same "
                         "softmax; reported as its own configuration")
    ap.add_argument("--score", choices=("sum", "headmax"), default="sum",
                    help="indexer score rule: heads summed into one query (default) or the best per-head "
                         "score (vector-ALU bound; reported as its own configuration)")
    ap.add_argument("--warm", action="store_true",
                    help="run the steps back to back; by default a 512 MB scratch buffer is read between "
                         "steps (cold last-level cache, as after a model's weights stream through it; no "
                         "dirty lines left to write back) and the step time comes from the events around "
                         "each step")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path (a batch would "
              "shard by sequence across GPUs with no exchange; one GPU's share is what this measures)",
              file=sys.stderr)
        sys.exit(2)
    if args.read_probe:
        read_probe(args)
        return
    if args.copy_probe:
        copy_probe()
        return
    if args.launch_floor:
        launch_floor(args)
        return
    if args.prefill:
        prefill_bench(args)
        return
    if args.prefill_write:
        prefill_write_bench(args)
        return

    import numpy as np

    import workloads as W

    w = W.WORKLOADS[args.workload]
    rule = 1 if args.score == "headmax" else 0
    # the oracle baseline first: its worker processes are forked before
    # anything touches the GPU
    cpu = None
    if args.cpu_only or not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.swa, args.cpu_threads, args.cpu_steps, rule)
    if args.cpu_only:
        print(json.dumps({"workload": w.name, "cpu_baseline": cpu}), flush=True)
        return

    import torch

    import fp4_compressed_sparse_amd as csa2

    csa2.load()
    torch.cuda.set_device(0)
    K, WU = args.steps, args.warmup
    total_steps = K + WU
    lengths = W.lengths(w)
    n_app = total_steps if w.append else 0
    capacity = int((int(lengths.max()) + n_app + 7) // 8 * 8)
    max_len = int(lengths.max()) + n_app
    t0 = time.perf_counter()
    caches = build_caches(w, lengths, capacity)
    for c in caches:
        c.max_len = max_len
    log(f"caches built in {time.perf_counter() - t0:.1f} s: {w.n_caches} x {w.batch} x {capacity} positions")

    B, H, L = w.batch, w.heads, len(w.pattern)
    lc = w.layer_caches()
    q_all = [[torch.from_numpy(W.queries(w.wid, l, s, B, H)).cuda() for l in range(L)]
             for s in range(total_steps)]
    rows_all = [torch.from_numpy(np.stack([W.append_rows(w.wid, c, s, B) for c in range(w.n_caches)])).cuda()
                if w.append else None for s in range(total_steps)]
    outs = [torch.zeros((B, H, 512), dtype=torch.float32, device="cuda") for _ in range(L)]
    # a Reuse layer's selection is its predecessor's: the driver forwards it
    # without a copy when both layers name the same buffer
    idxs = []
    for l, m in enumerate(w.pattern):
        idxs.append(idxs[-1] if m == 2 else torch.zeros((B, w.topk), dtype=torch.int32, device="cuda"))
    pool_out = torch.zeros((B, w.pool), dtype=torch.int32, device="cuda") if w.pool else None
    ws = csa2.workspace(B, H, max_len, w.pool, w.topk)
    rings, srows_all = [None] * L, [[None] * L for _ in range(total_steps)]
    if args.swa:
        # every layer's ring holds the last W positions of each sequence
        for l in range(L):
            rings[l] = csa2.SwaCache(B, args.swa)
            for b in range(B):
                n = int(lengths[b])
                lo = max(0, n - args.swa)
                x = torch.from_numpy(W.swa_rows(w.wid, l, b, lo, n - lo)).cuda()
                dst = torch.arange(lo, n, dtype=torch.int64, device="cuda") % args.swa + b * args.swa
                csa2.fp8_quantize_kv(x, rings[l].codes, rings[l].scales, dst_row=dst)
            rings[l].seq_len.copy_(torch.from_numpy(lengths.astype(np.int64)))
        srows_all = [[torch.from_numpy(W.swa_append_rows(w.wid, l, s, B)).cuda() for l in range(L)]
                     for s in range(total_steps)]
    plans = [csa2.StepPlan(caches, [(m, lc[l], q_all[s][l], outs[l], idxs[l], rings[l], srows_all[s][l])
                                    for l, m in enumerate(w.pattern)],
                           H, w.topk, w.pool, w.scale, ws, pool_out=pool_out, new_rows=rows_all[s], score=rule)
             for s in range(total_steps)]
    stream = torch.cuda.current_stream()

    for s in range(WU):
        plans[s].run(stream)
    torch.cuda.synchronize()
    assert csa2.device_error() == 0

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    hev = HipEvents()
    sev = [(hev.create(), hev.create()) for _ in range(K)]
    flush = None if args.warm else torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    flush_sink = torch.zeros((), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        if flush is not None:
            torch.sum(flush, dim=0, out=flush_sink)   # evicts the caches from the 256 MB MALL
        csa2.set_scan_events(*sev[i])
        ev[i][0].record(stream)
        plans[WU + i].run(stream)
        ev[i][1].record(stream)
    enqueued = time.perf_counter() - t_start      # host time to submit the K steps
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    csa2.set_scan_events(None, None)
    flags = csa2.device_error()
    if flags:
        log(f"device flags raised: {flags}")
        sys.exit(1)
    step_ms = [a.elapsed_time(b) for a, b in ev]
    scan_ms = [hev.elapsed_ms(a, b) for a, b in sev]
    for a, b in sev:
        hev.destroy(a)
        hev.destroy(b)

    ms_per_step = elapsed * 1e3 / K
    if flush is not None:                          # the flush reads are not part of a step
        ms_per_step = float(np.mean(step_ms))
        elapsed = ms_per_step * 1e-3 * K
    n_mid = [int(n) + (WU + K // 2 + 1 if w.append else 0) for n in lengths]
    uniq, touched = step_bytes(w, n_mid)
    if args.swa:                                   # every layer reads its own window (512 + 4 B per position)
        win_bytes = L * sum(min(args.swa, n) * 516 for n in n_mid)
        uniq, touched = uniq + win_bytes, touched + win_bytes
    scan_bytes = sum(n * TOKEN_BYTES for n in n_mid)
    scan_avg_s = float(np.mean(scan_ms)) * 1e-3
    achieved = scan_bytes / scan_avg_s / 1e9
    eff_gbs = uniq / (ms_per_step * 1e-3) / 1e9
    log(f"step: wall {ms_per_step * 1e3:.1f} us (host submit {enqueued * 1e6 / K:.1f} us), "
        f"events median {np.median(step_ms) * 1e3:.1f} us; "
        f"scan kernel avg {scan_avg_s * 1e6:.1f} us = {achieved:.0f} GB/s; "
        f"unique {uniq / 1e6:.1f} MB -> {eff_gbs:.0f} GB/s ({eff_gbs / PEAK_HBM_GBS * 100:.1f}% of peak); "
        f"touched {touched / 1e6:.1f} MB")

    result = {
        "metric": "CSA2 decode tokens/s + effective FP4 KV GB/s vs HBM peak (1M ctx, 1 GPU)",
        "value": round(B * K / elapsed, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": WU,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": B, "context": int(lengths.max()), "heads": H,
            "topk_blocks": w.topk, "pool_blocks": w.pool, "layers": L,
            "pattern": "[Full,Reindex,Reuse,Reuse,Reindex]x4" if w.wid == 3 else str(w.pattern),
            "kv_format": "FP4 E2M1 + E4M3/16ch, 288 B/position",
            "arithmetic": "indexer scores float32; attention on fp16 matrix-core operands with float32 accumulation",
            "effective_kv_gbs": round(eff_gbs, 1),
            "effective_kv_frac_of_peak": round(eff_gbs / PEAK_HBM_GBS, 4),
            "unique_kv_bytes_per_step": uniq, "touched_kv_bytes_per_step": touched,
            "median_event_step_us": round(float(np.median(step_ms)) * 1e3, 2),
            "mall_flush_between_steps": flush is not None,
            "swa_window": args.swa,
            "score_rule": args.score,
        },
        "roofline": {
            "bound": "hbm",
            # a batch scans its sequences' chunks laid end to end (scan_flat_kernel)
            "kernel": ("scan_flat_kernel" if 1 < B <= 512 else "scan_kernel") + " (first Full layer full-range scan)",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": pmc_traffic(PMC_FILE_FLAT if 1 < B <= 512 else PMC_FILE),
            "algorithmic_bytes_per_launch": scan_bytes,
            "avg_launch_us": round(scan_avg_s * 1e6, 2),
        },
    }
    if rule:
        # the per-head scan: H dot products of 512 unfused multiplies and 511
        # adds (plus the +0.0) per block, and the block key (8 rows x 512
        # multiply-adds, the x 1/8): vector-ALU bound
        nblk = sum((n + 7) // 8 for n in n_mid)
        ops = nblk * (H * 1024 + 8 * 512 * 2 + 512)
        tops = ops / scan_avg_s / 1e12
        result["roofline"] = {
            "bound": "alu",
            "kernel": "headmax_kernel (first Full layer per-head full-range scan)",
            "achieved": round(tops, 2),
            "peak": round(PEAK_VALU_TOPS, 2),
            "unit": "TFLOP/s",
            "frac": round(tops / PEAK_VALU_TOPS, 4),
            "traffic": None,
            "algorithmic_flops_per_launch": ops,
            "avg_launch_us": round(scan_avg_s * 1e6, 2),
        }
        log(f"per-head scan: {ops / 1e9:.2f} G float32 ops in {scan_avg_s * 1e6:.1f} us = {tops:.2f} T ops/s "
            f"({tops / PEAK_VALU_TOPS * 100:.1f}% of the {PEAK_VALU_TOPS:.1f} T ops/s unfused vector peak)")
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
