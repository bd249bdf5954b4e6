"""One workspace reused with different bounds: the words that must be zero
when a call starts move with the layout, so the library re-zeroes a
workspace whose previous call had another layout.  Checked with a caller
workspace (index_topk at batch 1, then batch 2 on the same buffer) and with
the library's own per-device workspace (decode_step_noalloc at batch 1, then
batch 2): pools and selections byte-equal to the oracle's."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
import workloads as W
from oracle import indexer as I
from oracle.select import select
from tests._gpu import cap_for, log, oracle_cache, require_gpu, to_device

pytestmark = pytest.mark.gpu


def _check_pool(oc, lengths, q, pool_out, idx, P, K):
    for b, n in enumerate(lengths):
        ids, sc = I.block_scores(oc.codes[b], oc.scales[b], n, q[b])
        assert np.array_equal(pool_out[b], select(ids, sc, P)), b
        assert np.array_equal(idx[b], select(ids, sc, K)), b


def test_caller_workspace_reused_with_another_batch():
    require_gpu()
    P, K, H = 256, 32, 16
    small = [9000]
    large = [20000, 12001]
    oc1 = oracle_cache(5, 0, small, cap_for(9000))
    oc2 = oracle_cache(5, 1, large, cap_for(20000))
    nbytes = max(csa2.workspace_bytes(1, H, 9000, P, K), csa2.workspace_bytes(2, H, 20000, P, K))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for oc, lengths in ((oc1, small), (oc2, large)):
            g = to_device(oc)
            q = W.queries(5, 7, rep, len(lengths), H)
            idx = torch.full((len(lengths), K), -7, dtype=torch.int32, device="cuda")
            pool = torch.full((len(lengths), P), -7, dtype=torch.int32, device="cuda")
            log(f"workspace reuse: rep {rep}, lengths {lengths}")
            csa2.index_topk(csa2.FULL, g, torch.from_numpy(q).cuda(), K, idx, ws, pool=P, pool_out=pool)
            torch.cuda.synchronize()
            _check_pool(oc, lengths, q, pool.cpu().numpy(), idx.cpu().numpy(), P, K)


def test_noalloc_with_changing_bounds():
    require_gpu()
    P, K, H = 512, 64, 16
    for lengths in ([9000], [20000, 12001], [9000]):
        oc = oracle_cache(5, 2, lengths, cap_for(max(lengths) + 1))
        g = to_device(oc, max_len=max(lengths) + 1)
        B = len(lengths)
        q = W.queries(5, 8, 0, B, H)
        out = torch.zeros((B, H, 512), dtype=torch.float32, device="cuda")
        idx = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
        pool = torch.full((B, P), -7, dtype=torch.int32, device="cuda")
        log(f"noalloc with changing bounds: lengths {lengths}")
        csa2.decode_step_noalloc([g], [(csa2.FULL, 0, torch.from_numpy(q).cuda(), out, idx)], H, K, P,
                                 1 / np.sqrt(512), pool_out=pool)
        torch.cuda.synchronize()
        assert csa2.device_error() == 0
        _check_pool(oc, lengths, q, pool.cpu().numpy(), idx.cpu().numpy(), P, K)
