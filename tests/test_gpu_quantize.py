"""GPU quantiser and append vs the oracle: codes and scales byte-equal."""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
import workloads as W
from oracle import formats as F
from oracle import quantize as Q
from tests._gpu import log, require_gpu

pytestmark = pytest.mark.gpu


def _edge_rows():
    """Rows that sit on every rounding boundary of both formats."""
    rows = []
    e4 = F.E4M3_TABLE[:0x7F].astype(np.float64)
    mids = (e4[:-1] + e4[1:]) / 2
    # amax exactly on 6 * every E4M3 midpoint, and one float32 ulp either side
    for k, m in enumerate(mids):
        a = np.float32(6 * m)
        for v in (a, np.nextafter(a, np.float32(0)), np.nextafter(a, np.float32(1e9))):
            r = np.zeros(Q.D, dtype=np.float32)
            r[(k % 32) * 16 + (k % 16)] = v if k % 3 else -v
            rows.append(r)
    # E2M1 ties: |x| = s * midpoint with s = 1 (amax = 6) and other scales
    for sb in (0x01, 0x07, 0x08, 0x30, 0x38, 0x3B, 0x55, 0x7E):
        s = F.e4m3_value(sb)
        r = np.zeros(Q.D, dtype=np.float32)
        for g in range(Q.NGROUPS):
            r[16 * g] = 6 * s
            for j, mid in enumerate(F.E2M1_MIDPOINTS):
                r[16 * g + 1 + j] = np.float32(s * mid) * (1 if j % 2 else -1)
                r[16 * g + 8 + j] = np.nextafter(np.float32(s * mid), np.float32(0))
        rows.append(r)
    # saturation, zeros, signed zeros, tiny values
    rows.append(np.full(Q.D, 3000.0, dtype=np.float32))
    rows.append(np.full(Q.D, -1e30, dtype=np.float32))
    rows.append(np.zeros(Q.D, dtype=np.float32))
    rows.append(-np.zeros(Q.D, dtype=np.float32))
    rows.append(np.full(Q.D, 1e-30, dtype=np.float32))
    rows.append(np.full(Q.D, 2.0 ** -10 * 6, dtype=np.float32))
    rng = np.random.default_rng(7)
    for _ in range(64):
        rows.append((rng.standard_normal(Q.D) * 2.0 ** rng.uniform(-24, 14, Q.D)).astype(np.float32))
    return np.stack(rows)


def _gpu_quantize(x, dst_row=None, dst_rows=None):
    n = dst_rows if dst_rows is not None else x.shape[0]
    codes = torch.full((n, Q.CODE_BYTES), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((n, Q.SCALE_BYTES), 0xCD, dtype=torch.uint8, device="cuda")
    xt = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    dr = None if dst_row is None else torch.from_numpy(dst_row).cuda()
    csa2.fp4_quantize_kv(xt, codes, scales, dst_row=dr)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def test_edge_rows_bit_exact():
    require_gpu()
    x = _edge_rows()
    log(f"quantize edge rows: {x.shape}")
    c, s = _gpu_quantize(x)
    oc, os_ = Q.quantize_rows(x)
    assert np.array_equal(s, os_), np.argwhere(s != os_)[:5]
    assert np.array_equal(c, oc), np.argwhere(c != oc)[:5]
    assert csa2.device_error() == 0


def test_workload_rows_bit_exact_and_ragged_count():
    require_gpu()
    x = W.kv_rows(4, 0, 3, 1000, 8191)          # odd row count: partial last workgroup
    c, s = _gpu_quantize(x)
    oc, os_ = Q.quantize_rows(x)
    assert np.array_equal(c, oc) and np.array_equal(s, os_)


def test_dst_rows_and_capacity_flag():
    require_gpu()
    x = W.kv_rows(4, 1, 0, 0, 64)
    perm = np.random.default_rng(3).permutation(100)[:64].astype(np.int64)
    perm[5] = 100          # out of range: skipped and flagged
    c, s = _gpu_quantize(x, dst_row=perm, dst_rows=100)
    oc, os_ = Q.quantize_rows(x)
    for i, d in enumerate(perm):
        if d < 100:
            assert np.array_equal(c[d], oc[i]) and np.array_equal(s[d], os_[i])
    untouched = sorted(set(range(100)) - set(perm.tolist()))
    assert np.all(c[untouched] == 0xAB)
    assert csa2.device_error() & csa2.FLAG_CAPACITY


def test_non_finite_group_flagged():
    require_gpu()
    x = W.kv_rows(4, 1, 0, 0, 4)
    x[1, 37] = np.inf
    x[2, 300] = np.nan
    c, s = _gpu_quantize(x)
    assert csa2.device_error() & csa2.FLAG_NONFINITE_KV
    assert np.all(c[1, 16:24] == 0) and s[1, 2] == 0
    assert np.all(c[2, 144:152] == 0) and s[2, 18] == 0
    oc, os_ = Q.quantize_rows(x[[0, 3]])
    assert np.array_equal(c[[0, 3]], oc) and np.array_equal(s[[0, 3]], os_)


def test_append_and_full_cache():
    require_gpu()
    cache = csa2.KVCache(3, 16)
    cache.seq_len.copy_(torch.tensor([0, 7, 16]))
    rows = W.append_rows(4, 0, 0, 3)
    csa2.append_kv(cache, torch.from_numpy(rows).cuda())
    torch.cuda.synchronize()
    assert cache.seq_len.cpu().tolist() == [1, 8, 16]
    assert csa2.device_error() & csa2.FLAG_CAPACITY
    oc, os_ = Q.quantize_rows(rows)
    codes, scales = cache.codes.cpu().numpy(), cache.scales.cpu().numpy()
    assert np.array_equal(codes[0, 0], oc[0]) and np.array_equal(scales[0, 0], os_[0])
    assert np.array_equal(codes[1, 7], oc[1]) and np.array_equal(scales[1, 7], os_[1])


def test_prefill_write_full_size():
    """The batch-64 prefill write: 16,384 fresh rows per sequence (1,048,576
    rows) in one launch; every 65,536-row chunk's codes and scales hash to
    the oracle's (tests/golden/prefill_write_1m.json, written by
    tests/golden/make_fullsize.py from the oracle alone)."""
    require_gpu()
    import hashlib
    import json
    import os
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "prefill_write_1m.json")) as f:
        gold = json.load(f)
    B, N = 64, W.PREFILL_WRITE_ROWS
    R, C = B * N, gold["chunk_rows"]
    assert gold["rows"] == R
    cache = csa2.KVCache(B, N)
    xs_all = W.kv_rows_threaded(4, 9, 0, R)              # sequence b = rows b*N .. b*N+N-1
    log("prefill write: rows generated")
    x = torch.from_numpy(xs_all).cuda()
    csa2.fp4_quantize_kv(x, cache.codes.view(-1, Q.CODE_BYTES), cache.scales.view(-1, Q.SCALE_BYTES))
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    codes = cache.codes.view(-1, Q.CODE_BYTES).cpu().numpy()
    scales = cache.scales.view(-1, Q.SCALE_BYTES).cpu().numpy()
    for k in range(R // C):
        assert hashlib.sha256(codes[k * C:(k + 1) * C].tobytes()).hexdigest() == gold["codes_sha256"][k], k
        assert hashlib.sha256(scales[k * C:(k + 1) * C].tobytes()).hexdigest() == gold["scales_sha256"][k], k
    log(f"prefill write: all {R} rows byte-equal to the oracle's")


def test_append_edge_rows_bit_exact():
    """csa2_append_kv on rows on every rounding boundary of both formats (one
    row per sequence, at varied positions): the decode-step append path runs
    the same quantiser as fp4_quantize_kv; bytes equal the oracle's."""
    require_gpu()
    x = _edge_rows()
    B = x.shape[0]
    log(f"append edge rows: {B} sequences")
    cache = csa2.KVCache(B, 16)
    start = (np.arange(B) * 5 % 9).astype(np.int64)              # positions 0..8
    cache.seq_len.copy_(torch.from_numpy(start))
    cache.codes.fill_(0xAB)
    cache.scales.fill_(0xCD)
    csa2.append_kv(cache, torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    assert np.array_equal(cache.seq_len.cpu().numpy(), start + 1)
    oc, os_ = Q.quantize_rows(x)
    codes, scales = cache.codes.cpu().numpy(), cache.scales.cpu().numpy()
    b = np.arange(B)
    assert np.array_equal(codes[b, start], oc), np.argwhere(codes[b, start] != oc)[:5]
    assert np.array_equal(scales[b, start], os_), np.argwhere(scales[b, start] != os_)[:5]
    other = np.ones((B, 16), dtype=bool)
    other[b, start] = False
    assert np.all(codes[other] == 0xAB) and np.all(scales[other] == 0xCD)


def test_decode_step_appends_edge_rows():
    """A decode step whose appended rows (two Full caches) are the edge rows:
    appended bytes equal the oracle's quantisation and every layer's
    selection equals the oracle's decode step on the same inputs.  Outputs
    are compared where the appended row lies in the latent's range (|x| <=
    sqrt(512), the bound the RMSNorm'd latent obeys): the attention rounds q
    to fp16, so a logit moves by up to 2^-11 * scale * sum_c |q_c k_c|, which
    for rows near the format maximum (2688 in every channel) is far outside
    the 2e-3 output bound, and inside it for rows of the latent's range."""
    require_gpu()
    from oracle.step import Cache, decode_step
    from tests._gpu import ATT_TOL, normwise_err
    x = _edge_rows()
    B, n0, H, K = x.shape[0], 21, 16, 2
    prefill = W.kv_rows(0, 0, 0, 0, n0)                           # the same 21 rows in every sequence
    pc, ps = Q.quantize_rows(prefill)
    ocs, gcs = [], []
    for c in range(2):
        oc = Cache(B, 24)
        oc.codes[:, :n0], oc.scales[:, :n0] = pc, ps
        oc.seq_len[:] = n0
        ocs.append(oc)
        g = csa2.KVCache(B, 24)
        g.codes.copy_(torch.from_numpy(oc.codes))
        g.scales.copy_(torch.from_numpy(oc.scales))
        g.seq_len.fill_(n0)
        g.max_len = n0 + 1
        gcs.append(g)
    rows = np.stack([x, x[::-1].copy()])                          # [2, B, 512]
    qs = [W.queries(0, l, 0, B, H) for l in range(3)]
    pattern = [(0, 0), (0, 1), (2, 1)]                            # Full, Full, Reuse
    ref = decode_step(ocs, [(m, c, qs[l]) for l, (m, c) in enumerate(pattern)], rows, K, 0, 1 / np.sqrt(512))
    outs = [torch.zeros((B, H, 512), dtype=torch.float32, device="cuda") for _ in range(3)]
    idxs = [torch.full((B, K), -9, dtype=torch.int32, device="cuda") for _ in range(3)]
    ws = csa2.workspace(B, H, n0 + 1, 0, K)
    csa2.decode_step(gcs, [(m, c, torch.from_numpy(qs[l]).cuda(), outs[l], idxs[l])
                           for l, (m, c) in enumerate(pattern)], H, K, 0, 1 / np.sqrt(512), ws,
                     new_rows=torch.from_numpy(rows).cuda())
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    for c in range(2):
        assert np.array_equal(gcs[c].seq_len.cpu().numpy(), np.full(B, n0 + 1))
        assert np.array_equal(gcs[c].codes.cpu().numpy(), ocs[c].codes), c
        assert np.array_equal(gcs[c].scales.cpu().numpy(), ocs[c].scales), c
    bound = np.sqrt(512.0)
    for l, (m, c) in enumerate(pattern):
        assert np.array_equal(idxs[l].cpu().numpy(), ref["idx"][l]), l
        ok = np.abs(rows[c]).max(axis=1) <= bound
        assert ok.sum() >= 100
        err = normwise_err(outs[l].cpu().numpy()[ok], ref["out"][l][ok])
        assert err <= ATT_TOL, (l, err)


def test_rows_beyond_one_grid_round():
    """More rows than one grid round covers (2^20 workgroups x 256 lanes =
    268,435,456 groups = 8,388,608 rows): the last 4,099 rows are quantised
    in a second grid-stride round.  65,536 workload rows, quantised once by
    the oracle, are tiled over the 8,392,707 rows; every row is compared."""
    require_gpu()
    S, R = 65536, 8_388_608 + 4_099
    src = W.kv_rows(4, 2, 0, 0, S)
    oc, os_ = Q.quantize_rows(src)
    log(f"quantize {R} rows (two grid rounds)")
    reps = (R + S - 1) // S
    x = torch.from_numpy(src).cuda().repeat(reps, 1)[:R]
    codes = torch.full((R, Q.CODE_BYTES), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((R, Q.SCALE_BYTES), 0xCD, dtype=torch.uint8, device="cuda")
    csa2.fp4_quantize_kv(x, codes, scales)
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    del x
    want_c = torch.from_numpy(oc).cuda()
    want_s = torch.from_numpy(os_).cuda()
    for r0 in range(0, R, S):
        n = min(S, R - r0)
        assert torch.equal(codes[r0:r0 + n], want_c[:n]), r0
        assert torch.equal(scales[r0:r0 + n], want_s[:n]), r0
