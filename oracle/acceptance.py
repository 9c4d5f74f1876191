"""Acceptance rules for comparing another implementation with the oracle
(test infrastructure).

Selected ids: let c1 >= c2 >= ... be the oracle's scores of the candidate
(non-recent) blocks. When (c16 - c17) / c16 >= rel, the other implementation's
16 must be the oracle's 16 exactly. Otherwise its set must contain every
candidate scoring above c16 * (1 + rel), and each remaining pick must score at
least c16 * (1 - rel). The recent block must always be present, ids must be
distinct, ascending and padded with -1 to topk + 1 entries; when every block
fits (nb <= topk + 1) all of them are selected.

Attention: max |a - b| <= 2e-2 and mean |a - b| <= 2e-3 against the oracle
evaluated on the other implementation's accepted ids, on identical FP8
operands.
"""
from __future__ import annotations

import numpy as np

REL = 1e-4
ATTN_MAX_ABS = 2e-2
ATTN_MEAN_ABS = 2e-3


def check_selection(bscores, ids, topk: int = 16, rel: float = REL):
    """Return None if `ids` is acceptable for the oracle block scores, else a message."""
    b = np.asarray(bscores, dtype=np.float64)
    ids = np.asarray(ids).astype(np.int64)
    nb = len(b)
    if ids.shape != (topk + 1,):
        return f"expected {topk + 1} ids, got shape {ids.shape}"
    if nb <= topk + 1:
        want = np.full(topk + 1, -1)
        want[:nb] = np.arange(nb)
        return None if np.array_equal(ids, want) else f"nb={nb}: expected all blocks, got {ids}"
    if np.any(ids < 0):
        return f"nb={nb}: padding present {ids}"
    if not np.all(np.diff(ids) > 0):
        return f"ids not strictly ascending: {ids}"
    if ids[-1] != nb - 1:
        return f"recent block {nb - 1} missing: {ids}"
    picks = ids[:-1]
    if np.any(picks >= nb - 1):
        return f"pick outside candidates: {ids}"
    cand = b[: nb - 1]
    srt = np.sort(cand)[::-1]
    c16, c17 = srt[topk - 1], srt[topk]
    order = np.lexsort((np.arange(nb - 1), -cand))
    exact = set(order[:topk].tolist())
    if c16 > 0 and (c16 - c17) / c16 >= rel:
        if set(picks.tolist()) != exact:
            return (f"clear gap ({(c16 - c17) / c16:.3g}): expected {sorted(exact)}, "
                    f"got {picks.tolist()}")
        return None
    must = set(np.nonzero(cand > c16 * (1 + rel))[0].tolist())
    if not must.issubset(set(picks.tolist())):
        return f"near tie: missing clear winners {sorted(must - set(picks.tolist()))}"
    low = [p for p in picks if cand[p] < c16 * (1 - rel)]
    if low:
        return f"near tie: picks {low} score below c16*(1-rel)"
    return None


def check_attention(out, ref, max_abs: float = ATTN_MAX_ABS, mean_abs: float = ATTN_MEAN_ABS):
    d = np.abs(np.asarray(out, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    if not np.all(np.isfinite(d)):
        return "non-finite output"
    if d.max() > max_abs or d.mean() > mean_abs:
        return f"attention error max {d.max():.3g} mean {d.mean():.3g}"
    return None
