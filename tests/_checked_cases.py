"""Cases of the checked-build comparison (tests/test_gpu_checked.py).

run_cases() runs a fixed set of calls through whichever library the binding
has loaded (the product libcsa2.so, or libcsa2_checked.so when CSA2_LIB_PATH
names it) and returns every output as numpy arrays, plus the device flag
word.  Inputs are seeded: random FP4 cache bytes with valid E4M3 scales,
workload queries and rows.  The cases reach every kernel: the quantisers,
the append, the single-sequence (up to 1,048,576 positions) and batched full scans, the pool select,
pool rescoring, both score rules, the decode attention with and without
in-kernel selection and window rows, the combines and the 64-head prefill
kernel, and the entry points on their own (selection, pool rescoring, score
export, attention).

As a script: python tests/_checked_cases.py OUT.npz (the child process of
the comparison test)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _cache(csa2, torch, rng, lengths, cap):
    B = len(lengths)
    g = csa2.KVCache(B, cap)
    codes = rng.integers(0, 256, size=(B, cap, 256), dtype=np.uint8)
    # E4M3 scales 2^-6 .. 2^0 (exponent fields 1..7): finite, never NaN
    scales = rng.integers(0x08, 0x40, size=(B, cap, 32), dtype=np.uint8)
    g.codes.copy_(torch.from_numpy(codes))
    g.scales.copy_(torch.from_numpy(scales))
    g.seq_len.copy_(torch.from_numpy(np.asarray(lengths, dtype=np.int64)))
    return g


def _steps(csa2, torch, W, res, tag, w, lengths, steps, window=0, score=0):
    rng = np.random.default_rng(1000 + w.wid + 7 * window + 13 * score)
    B, L, H = len(lengths), len(w.pattern), w.heads
    cap = int((max(lengths) + steps + 7) // 8 * 8)
    caches = [_cache(csa2, torch, rng, lengths, cap) for _ in range(w.n_caches)]
    for c in caches:
        c.max_len = int(max(lengths)) + steps
    rings = []
    for l in range(L if window else 0):
        ring = csa2.SwaCache(B, window)
        for b, n in enumerate(lengths):
            n = int(n)
            x = torch.from_numpy(W.swa_rows(w.wid, l, b, n - window, window)).cuda()
            dst = b * window + torch.arange(n - window, n, dtype=torch.int64, device="cuda") % window
            csa2.fp8_quantize_kv(x, ring.codes.view(B * window, 512), ring.scales.view(B * window), dst_row=dst)
        ring.seq_len.copy_(torch.from_numpy(np.asarray(lengths, dtype=np.int64)))
        rings.append(ring)
    q = [torch.zeros((B, H, 512), dtype=torch.float32, device="cuda") for _ in range(L)]
    outs = [torch.zeros((B, H, 512), dtype=torch.float32, device="cuda") for _ in range(L)]
    idxs = []
    for m in w.pattern:
        idxs.append(idxs[-1] if m == 2 else torch.zeros((B, w.topk), dtype=torch.int32, device="cuda"))
    rows = torch.zeros((w.n_caches, B, 512), dtype=torch.float32, device="cuda")
    srows = [torch.zeros((B, 512), dtype=torch.float32, device="cuda") for _ in range(L)]
    pool = torch.zeros((B, max(w.pool, 1)), dtype=torch.int32, device="cuda")
    ws = csa2.workspace(B, H, int(max(lengths)) + steps, w.pool, w.topk)
    lc = w.layer_caches()
    layers = [(m, lc[l], q[l], outs[l], idxs[l]) + ((rings[l], srows[l]) if window else ())
              for l, m in enumerate(w.pattern)]
    plan = csa2.StepPlan(caches, layers, H, w.topk, w.pool, w.scale, ws,
                         pool_out=pool if w.pool else None, new_rows=rows, score=score)
    for s in range(steps):
        for l in range(L):
            q[l].copy_(torch.from_numpy(W.queries(w.wid, l, s, B, H)))
            if window:
                srows[l].copy_(torch.from_numpy(W.swa_append_rows(w.wid, l, s, B)))
        rows.copy_(torch.from_numpy(np.stack([W.append_rows(w.wid, c, s, B) for c in range(w.n_caches)])))
        plan.run()
        torch.cuda.synchronize()
        if w.pool:
            res[f"{tag}/s{s}/pool"] = pool.cpu().numpy()
        for l in range(L):
            res[f"{tag}/s{s}/idx{l}"] = idxs[l].cpu().numpy()
            res[f"{tag}/s{s}/out{l}"] = outs[l].cpu().numpy()
    for c, cache in enumerate(caches):        # the appended rows and lengths
        res[f"{tag}/codes{c}"] = cache.codes.cpu().numpy()[:, -64:]
        res[f"{tag}/len{c}"] = cache.seq_len.cpu().numpy()
    for l, ring in enumerate(rings):
        res[f"{tag}/ring{l}"] = ring.codes.cpu().numpy()


def _prefill(csa2, torch, W, res, tag, n, qpos, heads, topk, seed):
    rng = np.random.default_rng(seed)
    g = _cache(csa2, torch, rng, [n], int((n + 7) // 8 * 8))
    g.max_len = n
    qpos = np.asarray(qpos, dtype=np.int64)
    T = qpos.size
    idx = np.full((T, topk), -1, dtype=np.int32)
    for t, p in enumerate(qpos):
        own = int(p) // 8
        k = min(topk - 1, own)
        pick = rng.choice(own, k, replace=False) if k else np.zeros(0, dtype=np.int64)
        sel = np.sort(np.concatenate([pick, [own]]))
        idx[t, :sel.size] = sel
    q = torch.from_numpy(W.queries(2, 7, seed, T, heads)).cuda()
    out = torch.zeros((T, heads, 512), dtype=torch.float32, device="cuda")
    ws = csa2.prefill_workspace(T, heads, topk)
    csa2.prefill_attend(g, 0, q, torch.from_numpy(qpos).cuda(), torch.from_numpy(idx).cuda(),
                        1 / np.sqrt(512), out, ws)
    torch.cuda.synchronize()
    res[f"{tag}/out"] = out.cpu().numpy()


def _standalone(csa2, torch, W, res):
    # the entry points on their own: a Full selection into a pool, pool
    # rescoring with its top-k, score export (every block and the pool's
    # blocks) and attention, under both score rules; batch 2, 70,000 and
    # 50,001 positions, 64 heads
    rng = np.random.default_rng(77)
    B, n, H = 2, 70000, 64
    g = _cache(csa2, torch, rng, [n, 50001], n)
    g.max_len = n
    q0 = torch.from_numpy(W.queries(2, 0, 0, B, H)).cuda()
    q1 = torch.from_numpy(W.queries(2, 1, 0, B, H)).cuda()
    for hm in (0, 1):
        ws = csa2.workspace(B, H, n, 2048, 256)
        idx0 = torch.full((B, 256), -7, dtype=torch.int32, device="cuda")
        pool = torch.full((B, 2048), -7, dtype=torch.int32, device="cuda")
        csa2.index_topk(csa2.FULL, g, q0, 256, idx0, ws, pool=2048, pool_out=pool, score=hm)
        idx1 = torch.full((B, 256), -7, dtype=torch.int32, device="cuda")
        csa2.index_topk(csa2.FULL, g, q1, 256, idx1, ws, cand=pool, score=hm)
        sc = torch.zeros((B, n // 8), dtype=torch.float32, device="cuda")
        csa2.block_scores(g, q0, sc, score=hm)
        scp = torch.zeros((B, 2048), dtype=torch.float32, device="cuda")
        csa2.block_scores(g, q1, scp, cand=pool, score=hm)
        out = torch.zeros((B, H, 512), dtype=torch.float32, device="cuda")
        csa2.sparse_attend(g, q1, idx1, 1 / np.sqrt(512), out, ws)
        torch.cuda.synchronize()
        for k, v in (("idx0", idx0), ("pool", pool), ("idx1", idx1), ("scores", sc), ("pool_scores", scp),
                     ("out", out)):
            res[f"alone{hm}/{k}"] = v.cpu().numpy()


def run_cases():
    import torch

    import fp4_compressed_sparse_amd as csa2
    import workloads as W

    csa2.load()
    torch.cuda.set_device(0)
    res = {}
    # quantisers: 5,000 FP4 rows into a permuted set of cache rows, 3,000 FP8 rows
    x = torch.from_numpy(W.kv_rows(0, 0, 0, 0, 5000)).cuda()
    dst = torch.from_numpy(np.random.default_rng(5).permutation(6000)[:5000].astype(np.int64)).cuda()
    codes = torch.zeros((6000, 256), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((6000, 32), dtype=torch.uint8, device="cuda")
    csa2.fp4_quantize_kv(x, codes, scales, dst_row=dst)
    c8 = torch.zeros((3000, 512), dtype=torch.uint8, device="cuda")
    s8 = torch.zeros(3000, dtype=torch.float32, device="cuda")
    csa2.fp8_quantize_kv(x[:3000], c8, s8)
    torch.cuda.synchronize()
    res["fp4/codes"], res["fp4/scales"] = codes.cpu().numpy(), scales.cpu().numpy()
    res["fp8/codes"], res["fp8/scales"] = c8.cpu().numpy(), s8.cpu().numpy()
    # 20 layers [F, Ri, Ru, Ru, Ri] x 4 at 20,000 positions, pool 2,048, 64 heads; with and without windows
    w3 = W.scaled(W.WORKLOADS[3], context=20000)
    _steps(csa2, torch, W, res, "w3", w3, [20000], 2)
    _steps(csa2, torch, W, res, "w3win", w3, [20000], 2, window=96)
    # the same 20 layers at 1,048,576 positions (the scan's dynamic schedule over all its work counters)
    _steps(csa2, torch, W, res, "w3full", W.WORKLOADS[3], [1 << 20], 2)
    # a ragged batch of 8 (3,000-60,000 positions): the batched scan, pool 2,048, 16 heads, top-128
    w4 = W.Workload(4, "ragged-b8", 8, 0, 16, 128, 2048, (0, 1, 2), 2, True)
    lens = np.random.default_rng(44).integers(3000, 60000, size=8)
    _steps(csa2, torch, W, res, "w4", w4, lens, 2)
    # the best-head score rule: [F, Ri, Ri] at 30,000 positions, pool 2,048, 64 heads
    w2 = W.scaled(W.WORKLOADS[2], context=30000)
    _steps(csa2, torch, W, res, "w2hm", w2, [30000], 1, score=1)
    # batch 4 without a pool: a Reindex layer that rescans
    w1 = W.scaled(W.WORKLOADS[1], context=9000)
    _steps(csa2, torch, W, res, "w1", w1, [9000] * 4, 1)
    # prefill: 64 heads (the eight-wave kernel, splits per query) and 16 heads
    _prefill(csa2, torch, W, res, "pre64", 12000, np.arange(12000 - 64, 12000), 64, 256, 12)
    _prefill(csa2, torch, W, res, "pre16", 4096, [0, 1, 7, 8, 63, 64, 200, 511, 1000, 4093, 4094, 4095],
             16, 64, 3)
    _standalone(csa2, torch, W, res)
    res["flags"] = np.asarray([csa2.device_error()], dtype=np.int64)
    return res


if __name__ == "__main__":
    import fp4_compressed_sparse_amd as _c
    print(f"library {_c.LIB_PATH}, CSA2_WG_ORDER={os.environ.get('CSA2_WG_ORDER', '')}", flush=True)
    out = run_cases()
    maps = open("/proc/self/maps").read()
    out["loaded_checked"] = np.asarray([int("libcsa2_checked.so" in maps)])
    np.savez(sys.argv[1], **out)
    print(f"{len(out)} arrays written", flush=True)
