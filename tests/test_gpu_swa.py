"""GPU local branch (FP8 sliding-window cache) vs the oracle.

Quantiser and ring append: bytes and scales bit-equal to the oracle's FP8
quantisation (ties, signed zeros, zero rows, power-of-two scalings, the
ring's wrap).  Attention with a window: within the 2e-3 normwise bound of
the oracle's float64 joint softmax, ring bytes uploaded from the oracle.
"""
import numpy as np
import pytest
import torch

import fp4_compressed_sparse_amd as csa2
import workloads as W
from oracle import swa as S
from oracle.formats import E4M3_TABLE
from tests._gpu import ATT_TOL, cap_for, log, normwise_err, oracle_cache, require_gpu, to_device

pytestmark = pytest.mark.gpu


def _rows_with_ties(n, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((n, 512)) * 2.0 ** rng.integers(-10, 10, (n, 1))).astype(np.float32)
    # rows whose scale is exactly 1 (amax 448): every midpoint of the E4M3
    # grid is an exact tie of the encoder
    mids = ((E4M3_TABLE[:0x7E] + E4M3_TABLE[1:0x7F]) / 2).astype(np.float32)
    for r in range(min(4, n)):
        x[r, :] = 0
        x[r, 0] = 448.0
        k = mids[rng.choice(mids.size, 300, replace=True)]
        x[r, 1:301] = k * np.where(rng.random(300) < 0.5, -1, 1).astype(np.float32)
    x[4, :8] = [448.0, 1.0, -0.5, 3.0, 0.3, 2.0 ** -10, 3 * 2.0 ** -10, 17.0]
    x[4, 8:] = 0
    x[5, :] = 0.0
    x[6, :] = -0.0
    x[6, 7] = 0.0
    x[7] = x[8] * np.float32(2.0 ** -20)               # tiny scale
    return x


def test_fp8_quantize_bit_exact():
    require_gpu()
    x = _rows_with_ties(300, 11)
    want_c, want_s = S.quantize_fp8_rows(x)
    codes = torch.full((300, 512), 0x55, dtype=torch.uint8, device="cuda")
    scales = torch.full((300,), -1.0, dtype=torch.float32, device="cuda")
    csa2.fp8_quantize_kv(torch.from_numpy(x).cuda(), codes, scales)
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    bad = np.argwhere(gc != want_c)
    assert bad.size == 0, (bad[:5], gc[tuple(bad[0])], want_c[tuple(bad[0])], x[bad[0][0], bad[0][1]])
    assert np.array_equal(gs.view(np.uint32), want_s.view(np.uint32))
    # destination rows: reversed order into a larger buffer
    dst = torch.arange(299, -1, -1, dtype=torch.int64, device="cuda") + 5
    codes2 = torch.zeros((310, 512), dtype=torch.uint8, device="cuda")
    scales2 = torch.zeros((310,), dtype=torch.float32, device="cuda")
    csa2.fp8_quantize_kv(torch.from_numpy(x).cuda(), codes2, scales2, dst_row=dst)
    torch.cuda.synchronize()
    assert np.array_equal(codes2.cpu().numpy()[5:305][::-1], want_c)
    assert np.array_equal(scales2.cpu().numpy()[5:305][::-1], want_s)
    log("fp8 quantiser: 300 rows bit-exact (ties, signed zeros, zero rows)")


def test_fp8_quantize_flags():
    require_gpu()
    x = W.swa_rows(0, 0, 0, 0, 3)
    x[1, 7] = np.nan
    x[2, 9] = 70000.0
    codes = torch.zeros((3, 512), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((3,), dtype=torch.float32, device="cuda")
    csa2.device_error()                                   # clear
    csa2.fp8_quantize_kv(torch.from_numpy(x).cuda(), codes, scales)
    torch.cuda.synchronize()
    flags = csa2.device_error()
    assert flags & csa2.FLAG_NONFINITE_KV and flags & csa2.FLAG_SWA_RANGE
    assert np.all(codes.cpu().numpy()[1] == 0) and scales.cpu().numpy()[1] == 0
    want_c, want_s = S.quantize_fp8_rows(x[2:3])
    assert np.array_equal(codes.cpu().numpy()[2], want_c[0]) and scales.cpu().numpy()[2] == want_s[0]


def test_ring_append_wraps():
    require_gpu()
    B, Wn, steps = 3, 48, 70
    start = np.array([0, 47, 100], dtype=np.int64)
    ring = csa2.SwaCache(B, Wn)
    ring.seq_len.copy_(torch.from_numpy(start))
    hist = {b: {} for b in range(B)}
    for t in range(steps):
        rows = W.swa_append_rows(1, 0, t, B)
        csa2.swa_append(ring, torch.from_numpy(rows).cuda())
        c8, s8 = S.quantize_fp8_rows(rows)
        for b in range(B):
            hist[b][int(start[b]) + t] = (c8[b], s8[b])
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    assert np.array_equal(ring.seq_len.cpu().numpy(), start + steps)
    gc, gs = ring.codes.cpu().numpy(), ring.scales.cpu().numpy()
    for b in range(B):
        L = int(start[b]) + steps
        for p in range(L - Wn, L):
            c, s = hist[b][p]
            assert np.array_equal(gc[b, p % Wn], c), (b, p)
            assert gs[b, p % Wn] == s
    log(f"ring append: {steps} steps into window {Wn}, wrapped slots bit-exact")


def oracle_swa(wid, layer, lengths, window, capacity):
    """Oracle SWA cache holding the last `window` positions of each sequence."""
    sw = S.SwaCache(len(lengths), capacity)
    for b, n in enumerate(lengths):
        lo = max(0, int(n) - window)
        if n > lo:
            sw.write(b, lo, W.swa_rows(wid, layer, b, lo, int(n) - lo))
        sw.seq_len[b] = n
    return sw


def ring_to_device(sw, window):
    """GPU ring holding the oracle's bytes of each sequence's window."""
    B = sw.batch
    ring = csa2.SwaCache(B, window)
    codes = np.zeros((B, window, 512), dtype=np.uint8)
    scales = np.zeros((B, window), dtype=np.float32)
    for b in range(B):
        for p in S.window_positions(sw.seq_len[b], window):
            codes[b, p % window] = sw.codes[b, p]
            scales[b, p % window] = sw.scales[b, p]
    ring.codes.copy_(torch.from_numpy(codes))
    ring.scales.copy_(torch.from_numpy(scales))
    ring.seq_len.copy_(torch.from_numpy(sw.seq_len))
    return ring


@pytest.mark.parametrize("heads,topk,window,lengths,swa_lengths", [
    (16, 64, 128, [4096 + 5, 2000, 3], [4096 + 5, 2000, 3]),
    (64, 256, 128, [3000], [3000]),
    (32, 100, 100, [2500, 900], [60, 2500]),          # window not a multiple of 64, a short ring
    (64, 64, 1024, [5000, 1], [5000, 1]),             # largest window
    (16, 8, 300, [700, 0], [700, 0]),                 # empty sequence and empty ring
])
def test_attend_with_window_matches_oracle(heads, topk, window, lengths, swa_lengths):
    require_gpu()
    oc = oracle_cache(3, 0, lengths, cap_for(max(lengths)))
    g = to_device(oc)
    sw = oracle_swa(3, 1, swa_lengths, window, max(swa_lengths) + 1)
    ring = ring_to_device(sw, window)
    B = len(lengths)
    q = W.queries(3, 4, heads, B, heads)
    rng = np.random.default_rng(heads + window)
    idx = np.full((B, topk), -1, dtype=np.int32)
    for b, n in enumerate(lengths):
        nb = (n + 7) // 8
        k = min(topk, nb)
        if k:
            idx[b, :k] = np.sort(rng.choice(nb, k, replace=False))
    scale = 1 / np.sqrt(512)
    ws = csa2.workspace(B, heads, g.max_len, 0, topk)
    out = torch.full((B, heads, 512), 9.0, dtype=torch.float32, device="cuda")
    log(f"attend+window heads={heads} topk={topk} window={window} lengths={lengths} ring={swa_lengths}")
    csa2.sparse_attend(g, torch.from_numpy(q).cuda(), torch.from_numpy(idx).cuda(), scale, out, ws, swa=ring)
    torch.cuda.synchronize()
    assert csa2.device_error() == 0
    got = out.cpu().numpy()
    ref = np.stack([S.attend_with_window(oc.codes[b], oc.scales[b], n, q[b], idx[b], scale,
                                         sw.codes[b], sw.scales[b], swa_lengths[b], window)
                    for b, n in enumerate(lengths)])
    err = normwise_err(got, ref)
    log(f"  normwise error {err:.2e}")
    assert err <= ATT_TOL
