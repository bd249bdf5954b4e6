"""GPU sparse attention vs the oracle's float64 attention (max normwise
relative error <= 2e-3 per (sequence, head) row)."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
import workloads as W
from oracle.attend import sparse_attend
from tests._gpu import ATT_TOL, cap_for, log, normwise_err, oracle_cache, require_gpu, to_device

pytestmark = pytest.mark.gpu


def _attend(g, q, idx, scale, ws=None):
    B, H = q.shape[:2]
    topk = idx.shape[1]
    ws = ws if ws is not None else csa2.workspace(B, H, g.max_len, 0, topk)
    out = torch.full((B, H, 512), 9.0, dtype=torch.float32, device="cuda")
    csa2.sparse_attend(g, torch.from_numpy(q).cuda(), torch.from_numpy(idx).cuda(), scale, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# (16, 400): 50 splits per head tile (two-wave combine, one batch);
# (16, 1024): 128 splits (two-wave combine, two batches)
@pytest.mark.parametrize("heads,topk", [(16, 64), (32, 100), (64, 256), (16, 128), (16, 400), (16, 1024)])
def test_attend_matches_oracle(heads, topk):
    require_gpu()
    lengths = [4096 + 5, 2000, 3]
    oc = oracle_cache(3, 0, lengths, cap_for(4101))
    g = to_device(oc)
    q = W.queries(3, 1, heads, len(lengths), heads)
    rng = np.random.default_rng(heads + topk)
    idx = np.full((len(lengths), topk), -1, dtype=np.int32)
    for b, n in enumerate(lengths):
        nb = (n + 7) // 8
        k = min(topk, nb)
        idx[b, :k] = np.sort(rng.choice(nb, k, replace=False))
    idx[0, 3] = -1                          # a hole inside the list
    log(f"attend heads={heads} topk={topk}")
    got = _attend(g, q, idx, 1 / np.sqrt(512))
    ref = np.stack([sparse_attend(oc.codes[b], oc.scales[b], n, q[b], idx[b], 1 / np.sqrt(512))
                    for b, n in enumerate(lengths)])
    err = normwise_err(got, ref)
    log(f"  normwise error {err:.2e}")
    assert err <= ATT_TOL


def test_attend_edge_cases():
    require_gpu()
    lengths = [1, 0, 16]
    oc = oracle_cache(3, 1, lengths, 16)
    g = to_device(oc)
    q = W.queries(3, 2, 0, 3, 16)
    idx = np.array([[0, -1], [-1, -1], [1, 1]], dtype=np.int32)   # duplicate block in row 2
    got = _attend(g, q, idx, 0.3)
    ref0 = sparse_attend(oc.codes[0], oc.scales[0], 1, q[0], idx[0], 0.3)
    assert normwise_err(got[0], ref0) <= 1e-6          # one position: the row itself
    assert np.all(got[1] == 0)                          # nothing selected
    # a repeated block counts twice, as the definition gathers it twice
    ref2 = sparse_attend(oc.codes[2], oc.scales[2], 16, q[2], idx[2], 0.3)
    assert normwise_err(got[2], ref2) <= ATT_TOL
