"""Top-k block selection (oracle; test infrastructure only).

CSA2 keeps the top-k most relevant positions [P2 "same notes, many layers"],
here at block granularity.  The pages give no tie rule; ties go to the
lowest block id.  The selected set is returned in ascending id order (it is a
set; the order carries no meaning) and padded with -1 when there are fewer
than k candidates.
"""
import numpy as np


def select(ids, scores, k):
    """Top-min(k, len(ids)) of (score descending, id ascending), sorted by id.

    ids: int [m] candidate block ids (distinct); scores: float32 [m].
    Returns int32 [k], ascending ids then -1 padding.
    """
    ids = np.asarray(ids, dtype=np.int64)
    scores = np.asarray(scores, dtype=np.float32)
    if ids.shape != scores.shape:
        raise ValueError("ids and scores differ in shape")
    if np.any(np.isnan(scores)):
        raise ValueError("NaN score")
    order = sorted(range(ids.size), key=lambda i: (-float(scores[i]), int(ids[i])))
    take = sorted(int(ids[i]) for i in order[:min(k, ids.size)])
    out = np.full(k, -1, dtype=np.int32)
    out[:len(take)] = take
    return out
