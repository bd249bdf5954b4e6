"""A decode step captured as a HIP graph (torch.cuda.graph) and replayed:
every replay, with the program's own eager copies of the next step's
inputs between replays, gives bit-identical selections, pool and outputs to
the same step run eagerly on an identical copy of the caches.  The step
leaves its workspace counters at zero with kernels (no memset nodes), which
is what makes a captured step replayable."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
import workloads as W
from tests._gpu import cap_for, log, oracle_cache, require_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("window", [0, 96])
def test_captured_step_replays_match_eager(window):
    require_gpu()
    w = W.scaled(W.WORKLOADS[3], context=20000)        # 20 layers, pool 2,048 (fused selection)
    n0, steps, B = 20000 - 3, 3, 1
    L, H = len(w.pattern), w.heads
    lc = w.layer_caches()
    cap = cap_for(n0, steps)

    def make():
        caches = [to_device(oracle_cache(w.wid, c, [n0], cap), max_len=n0 + steps) for c in range(w.n_caches)]
        rings = []
        for l in range(L if window else 0):
            ring = csa2.SwaCache(B, window)
            x = torch.from_numpy(W.swa_rows(w.wid, l, 0, n0 - window, window)).cuda()
            dst = torch.arange(n0 - window, n0, dtype=torch.int64, device="cuda") % window
            csa2.fp8_quantize_kv(x, ring.codes, ring.scales, dst_row=dst)
            ring.seq_len.fill_(n0)
            rings.append(ring)
        q = [torch.zeros((B, H, 512), dtype=torch.float32, device="cuda") for _ in range(L)]
        outs = [torch.zeros((B, H, 512), dtype=torch.float32, device="cuda") for _ in range(L)]
        idxs = []
        for m in w.pattern:
            idxs.append(idxs[-1] if m == 2 else torch.zeros((B, w.topk), dtype=torch.int32, device="cuda"))
        rows = torch.zeros((w.n_caches, B, 512), dtype=torch.float32, device="cuda")
        srows = [torch.zeros((B, 512), dtype=torch.float32, device="cuda") for _ in range(L)]
        pool = torch.zeros((B, w.pool), dtype=torch.int32, device="cuda")
        ws = csa2.workspace(B, H, n0 + steps, w.pool, w.topk)
        layers = [(m, lc[l], q[l], outs[l], idxs[l]) + ((rings[l], srows[l]) if window else ())
                  for l, m in enumerate(w.pattern)]
        plan = csa2.StepPlan(caches, layers, H, w.topk, w.pool, w.scale, ws, pool_out=pool, new_rows=rows)
        return plan, q, rows, srows, outs, idxs, pool

    def feed(q, rows, srows, s):
        for l in range(L):
            q[l].copy_(torch.from_numpy(W.queries(w.wid, l, s, B, H)))
            if window:
                srows[l].copy_(torch.from_numpy(W.swa_append_rows(w.wid, l, s, B)))
        rows.copy_(torch.from_numpy(np.stack([W.append_rows(w.wid, c, s, B) for c in range(w.n_caches)])))

    eager = make()
    graph_side = make()
    torch.cuda.synchronize()
    ref = []
    for s in range(steps):
        plan, q, rows, srows, outs, idxs, pool = eager
        feed(q, rows, srows, s)
        plan.run()
        torch.cuda.synchronize()
        ref.append(([o.clone() for o in outs], [i.clone() for i in idxs], pool.clone()))
    assert csa2.device_error() == 0

    plan, q, rows, srows, outs, idxs, pool = graph_side
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            plan.run(stream)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    # capture records the step without running it: the caches are untouched
    for s in range(steps):
        feed(q, rows, srows, s)                         # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        r_outs, r_idxs, r_pool = ref[s]
        assert torch.equal(pool, r_pool), s
        for l in range(L):
            assert torch.equal(idxs[l], r_idxs[l]), (s, l)
            assert torch.equal(outs[l], r_outs[l]), (s, l)
        log(f"replay {s} (window {window}): pool, {L} selections and outputs bit-identical to eager")
    assert csa2.device_error() == 0
