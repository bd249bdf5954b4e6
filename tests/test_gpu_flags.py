"""Device flags of the decode path: each data-dependent problem the header
names raises its bit in csa2_device_error, and the call still completes with
the offending item skipped (the rest compared with the oracle)."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
import workloads as W
from oracle.attend import sparse_attend
from tests._gpu import ATT_TOL, cap_for, normwise_err, oracle_cache, require_gpu, to_device

pytestmark = pytest.mark.gpu

LENGTHS = [300, 100]


def _cache():
    oc = oracle_cache(3, 4, LENGTHS, cap_for(max(LENGTHS)))
    return oc, to_device(oc)


def test_nonfinite_query_flags_in_index():
    """A NaN in one query head reaches the indexer's head sum: FLAG_NONFINITE_Q."""
    require_gpu()
    _, g = _cache()
    q = W.queries(3, 7, 0, len(LENGTHS), 16)
    q[1, 5, 77] = np.nan
    topk = 4
    idx = torch.full((len(LENGTHS), topk), -9, dtype=torch.int32, device="cuda")
    ws = csa2.workspace(len(LENGTHS), 16, g.max_len, 0, topk)
    assert csa2.device_error() == 0
    csa2.index_topk(csa2.FULL, g, torch.from_numpy(q).cuda(), topk, idx, ws)
    assert csa2.device_error() & csa2.FLAG_NONFINITE_Q


def test_bad_candidate_flags_in_rescoring():
    """A candidate block past the sequence's end: FLAG_BAD_INDEX; it is never selected."""
    require_gpu()
    _, g = _cache()
    q = torch.from_numpy(W.queries(3, 8, 0, len(LENGTHS), 16)).cuda()
    nb = (np.array(LENGTHS) + 7) // 8
    cand = np.stack([np.arange(16), np.arange(16)]).astype(np.int32)
    cand[1, 15] = int(nb[1]) + 3                         # past sequence 1's 13 blocks
    idx = torch.full((2, 16), -9, dtype=torch.int32, device="cuda")
    ws = csa2.workspace(2, 16, g.max_len, 0, 16)
    assert csa2.device_error() == 0
    csa2.index_topk(csa2.REINDEX, g, q, 16, idx, ws, cand=torch.from_numpy(cand).cuda())
    assert csa2.device_error() & csa2.FLAG_BAD_INDEX
    got = idx.cpu().numpy()
    assert int(nb[1]) + 3 not in got[1].tolist()


def test_bad_index_flags_in_attention_and_is_skipped():
    """A selected block past the sequence's end in csa2_sparse_attend:
    FLAG_BAD_INDEX, and the output equals attention without that block."""
    require_gpu()
    oc, g = _cache()
    q = W.queries(3, 9, 0, len(LENGTHS), 16)
    idx = np.array([[0, 5, 9, 37], [1, 2, 12, 40]], dtype=np.int32)   # 40 >= 13 blocks of sequence 1
    out = torch.full((2, 16, 512), 7.0, dtype=torch.float32, device="cuda")
    ws = csa2.workspace(2, 16, g.max_len, 0, 4)
    assert csa2.device_error() == 0
    csa2.sparse_attend(g, torch.from_numpy(q).cuda(), torch.from_numpy(idx).cuda(), 1 / np.sqrt(512), out, ws)
    assert csa2.device_error() & csa2.FLAG_BAD_INDEX
    valid = idx.copy()
    valid[1, 3] = -1
    ref = np.stack([sparse_attend(oc.codes[b], oc.scales[b], n, q[b], valid[b], 1 / np.sqrt(512))
                    for b, n in enumerate(LENGTHS)])
    assert normwise_err(out.cpu().numpy(), ref) <= ATT_TOL


def test_query_outside_fp16_range_flags():
    """A query value with no fp16 value (|q| >= 65520) in the attention: FLAG_Q_RANGE."""
    require_gpu()
    _, g = _cache()
    q = W.queries(3, 10, 0, len(LENGTHS), 16)
    idx = np.array([[0, 1], [0, 1]], dtype=np.int32)
    out = torch.zeros((2, 16, 512), dtype=torch.float32, device="cuda")
    ws = csa2.workspace(2, 16, g.max_len, 0, 2)
    assert csa2.device_error() == 0
    csa2.sparse_attend(g, torch.from_numpy(q).cuda(), torch.from_numpy(idx).cuda(), 0.04, out, ws)
    assert csa2.device_error() == 0                      # in range: no flag
    q[0, 3, 100] = 70000.0
    csa2.sparse_attend(g, torch.from_numpy(q).cuda(), torch.from_numpy(idx).cuda(), 0.04, out, ws)
    assert csa2.device_error() & csa2.FLAG_Q_RANGE
