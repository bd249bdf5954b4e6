"""Sparse softmax attention over the selected positions (oracle; test only).

CSA2 attends only to the selected history positions [P2 "same notes, many
layers"].  The cached latent is 512 channels [P3 section 三] and is
dequantised where it is used [P1 section 五].

Readings (the pages do not spell out the attention):
  * Every head attends over the same gathered positions; keys and values are
    both the dequantised 512-channel latent (V = K), shared by all heads.
  * Positions are 8b+t for each selected block b >= 0, t = 0..7, that are
    below the sequence length n (n counts the position appended this step).
  * logits z_p = scale * (q_h . k_p) (scale = 1/sqrt(512) in every workload),
    w = softmax(z), o_h = sum_p w_p v_p, all in float64.
  * No selected position gives o_h = 0.
"""
import numpy as np

from .indexer import BLOCK
from .quantize import D, dequantize_rows


def gather_positions(idx, n):
    pos = []
    for b in np.asarray(idx).tolist():
        if b < 0:
            continue
        for t in range(BLOCK):
            p = BLOCK * b + t
            if p < n:
                pos.append(p)
    return np.asarray(pos, dtype=np.int64)


def sparse_attend(codes, scales, n, q, idx, scale):
    """One sequence: q float32 [H, 512], idx int [K] -> float64 [H, 512]."""
    q = np.asarray(q, dtype=np.float64)
    pos = gather_positions(idx, n)
    if pos.size == 0:
        return np.zeros((q.shape[0], D), dtype=np.float64)
    kv = dequantize_rows(codes[pos], scales[pos]).astype(np.float64)   # [P, 512]
    z = (q @ kv.T) * float(scale)                                       # [H, P]
    z = z - z.max(axis=1, keepdims=True)
    w = np.exp(z)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ kv
