"""Sliding-window local branch with an FP8 KV cache (oracle; test
infrastructure only).

Local context is handled by sliding-window attention: each position looks
at a stretch of recent positions [P2 "halve the long input"].  Entries older
than the window are never read by the current decode step [P1 section 三].
The main (global) KV moved from FP8 to FP4, while the SWA KV, being more
sensitive to quantisation, stays FP8 [P2 "same notes, many layers"].

Readings (the pages give no window size, FP8 layout or merge rule):
  * FP8 is OCP E4M3FN (the variant the FP4 path's scales already use).  One
    float32 scale per position: s = fl32(amax / 448) of the row's largest
    magnitude; each value becomes the E4M3 code nearest to fl32(x / s)
    (ties to the even code, saturating at 448) with its sign bit kept;
    s == 0 gives magnitude 0.  A row is 512 code bytes + 4 scale bytes.
  * The window of a sequence with L positions is positions
    max(0, L - W) .. L - 1, the current token's own position included, for a
    window size W that is a model constant.
  * Every decoder layer has its own SWA KV (one row per position per layer),
    written for the new token before the layer attends.
  * The two branches form one softmax: the keys of the CSA2-selected
    positions (FP4 global KV) and of the window positions (FP8 SWA KV) are
    attended together with the same logit scale; keys = values in both
    caches.  Equivalently, each branch's (max, sum, weighted sum) is merged
    by log-sum-exp.
"""
import numpy as np

from .attend import gather_positions
from .formats import E4M3_MIDPOINTS, E4M3_TABLE, _rne_index
from .quantize import D, dequantize_rows

E4M3_MAX = 448.0
SWA_ROW_BYTES = D + 4          # 512 E4M3 codes + one float32 scale


def e4m3_code(y):
    """E4M3FN bytes of float values y: RNE to the nearest code, ties to the
    even code, saturating at 448, sign bit kept (also for -0 and for values
    that round to zero).  Exact: the midpoints and y are exact in float64."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(~np.isfinite(y)):
        raise ValueError("non-finite value")
    mag = _rne_index(np.abs(y), E4M3_MIDPOINTS).astype(np.uint8)   # 0x00..0x7E
    return (np.signbit(y).astype(np.uint8) << 7) | mag


def quantize_fp8_rows(x):
    """float32 [R, 512] -> (codes uint8 [R, 512], scales float32 [R]).

    Raises ValueError on non-finite input.
    """
    x = np.asarray(x)
    if x.dtype != np.float32 or x.ndim != 2 or x.shape[1] != D:
        raise ValueError("expected float32 [R, 512]")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input row")
    amax = np.abs(x).max(axis=1)                                   # exact
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)           # IEEE float32 division
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    y = (x / safe[:, None]).astype(np.float32)                     # IEEE float32 division
    codes = e4m3_code(y)
    codes = np.where(s[:, None] > 0, codes, codes & 0x80).astype(np.uint8)
    return codes, s


def dequantize_fp8_rows(codes, scales):
    """(codes [R, 512], scales [R]) -> float64 [R, 512], exact (a 4-bit
    significand times a float32 scale fits float64)."""
    v = E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
    if np.any(np.isnan(v)):
        raise ValueError("NaN code in SWA cache")
    return v * np.asarray(scales, dtype=np.float64)[..., None]


def window_positions(length, window):
    """Positions the window of a sequence of `length` positions covers."""
    length, window = int(length), int(window)
    return np.arange(max(0, length - window), length, dtype=np.int64)


def attend_with_window(codes, scales, n, q, idx, scale, swa_codes, swa_scales, swa_len, window):
    """One sequence, both branches in one softmax -> float64 [H, 512].

    codes/scales/n/idx: the FP4 global cache and this layer's block
    selection (as in the sparse attention); swa_codes [P, 512] and
    swa_scales [P] hold the FP8 SWA rows by position, swa_len positions of
    which exist; window: the window size (0 = no local branch).
    """
    q = np.asarray(q, dtype=np.float64)
    keys = []
    pos = gather_positions(idx, n)
    if pos.size:
        keys.append(dequantize_rows(codes[pos], scales[pos]).astype(np.float64))
    wpos = window_positions(swa_len, window)
    if wpos.size:
        keys.append(dequantize_fp8_rows(swa_codes[wpos], swa_scales[wpos]))
    if not keys:
        return np.zeros((q.shape[0], D), dtype=np.float64)
    kv = np.concatenate(keys, axis=0)                               # [P, 512]
    z = (q @ kv.T) * float(scale)
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ kv


class SwaCache:
    """One layer's FP8 SWA cache for a batch of sequences, kept by position
    (the oracle stores every position; only the window is ever read)."""

    def __init__(self, batch, capacity):
        self.codes = np.zeros((batch, capacity, D), dtype=np.uint8)
        self.scales = np.zeros((batch, capacity), dtype=np.float32)
        self.seq_len = np.zeros(batch, dtype=np.int64)

    @property
    def batch(self):
        return self.codes.shape[0]

    def write(self, b, start, rows):
        rows = np.asarray(rows, dtype=np.float32).reshape(-1, D)
        if start + rows.shape[0] > self.codes.shape[1]:
            raise ValueError("SWA capacity exceeded")
        c, s = quantize_fp8_rows(rows)
        self.codes[b, start:start + rows.shape[0]] = c
        self.scales[b, start:start + rows.shape[0]] = s

    def append(self, rows):
        """One row per sequence (float32 [B, 512]) at position seq_len[b]."""
        rows = np.asarray(rows, dtype=np.float32).reshape(self.batch, D)
        for b in range(self.batch):
            self.write(b, int(self.seq_len[b]), rows[b:b + 1])
            self.seq_len[b] += 1


__all__ = ["e4m3_code", "quantize_fp8_rows", "dequantize_fp8_rows", "window_positions",
           "attend_with_window", "SwaCache", "SWA_ROW_BYTES"]
