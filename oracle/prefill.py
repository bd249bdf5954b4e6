"""Batched prefill-side sparse attention (oracle; test infrastructure only).

The pages put the cost of long inputs in the prefill [P2 introduction and
the section on the encoder-decoder split] and describe the sparse attention
only for the decode path [P2 "same notes, many layers"].  Reading taken for
the prefill side: a chunk of T queries of one sequence, query t at cache
position qpos[t], each with its own selection of blocks idx[t]; query t
attends causally, to the selected positions p <= qpos[t] (its own position
included, as the decode step includes the position it appends), with the
same arithmetic as the decode attention (oracle.attend.sparse_attend).
With a local branch (oracle/swa.py) each position looks at its own nearby
stretch [P2 "halve the long input"]: query t's window is the `window`
positions ending at qpos[t], joined to its sparse positions in one softmax,
as at a decode step whose sequence ends at qpos[t].
"""
import numpy as np

from .attend import sparse_attend
from .quantize import D
from .swa import attend_with_window


def prefill_attend(codes, scales, qpos, q, idx, scale, swa_codes=None, swa_scales=None, window=0):
    """codes/scales: one sequence's cache rows; qpos int [T]; q float32
    [T, H, 512]; idx int [T, K] -> float64 [T, H, 512].  swa_codes [P, 512]
    / swa_scales [P]: the sequence's FP8 SWA rows by position (window > 0)."""
    qpos = np.asarray(qpos, dtype=np.int64)
    q = np.asarray(q)
    out = np.zeros((q.shape[0], q.shape[1], D), dtype=np.float64)
    for t in range(q.shape[0]):
        n = int(qpos[t]) + 1
        if window:
            out[t] = attend_with_window(codes, scales, n, q[t], idx[t], scale, swa_codes, swa_scales, n, window)
        else:
            out[t] = sparse_attend(codes, scales, n, q[t], idx[t], scale)
    return out
