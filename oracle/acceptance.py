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

Rounded encodings (the cache-insertion path, whose E4M3 and NVFP4 decisions
are taken on fp32 values that differ from the oracle's fp64 values by
rounding): a byte is accepted when it is the encoding of some value within
delta of the oracle's; delta = 0 demands equality.
"""
from __future__ import annotations

import numpy as np

from .formats import E2M1_MID, E4M3_MID, E4M3_POS, e4m3_encode, nearest_even_index
from .nvfp4 import GROUP, unpack_nibbles

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


def attention_error(out, ref):
    """(max |out - ref|, mean |out - ref|) over every element, in float64;
    (inf, inf) when either side holds a non-finite value or the shapes differ."""
    a = np.asarray(out, dtype=np.float64)
    b = np.asarray(ref, dtype=np.float64)
    if a.shape != b.shape or a.size == 0:
        return float("inf"), float("inf")
    d = np.abs(a - b)
    if not np.all(np.isfinite(d)):
        return float("inf"), float("inf")
    return float(d.max()), float(d.mean())


def check_attention(out, ref, max_abs: float = ATTN_MAX_ABS, mean_abs: float = ATTN_MEAN_ABS):
    """None when out is within both bars of ref (max-abs AND mean-abs error),
    else a message. Non-finite values and shape mismatches always fail."""
    a = np.asarray(out, dtype=np.float64)
    b = np.asarray(ref, dtype=np.float64)
    if a.shape != b.shape or a.size == 0:
        return f"attention shape {a.shape} vs oracle {b.shape}"
    mx, mean = attention_error(a, b)
    if not np.isfinite(mx):
        return "non-finite output"
    if mx > max_abs or mean > mean_abs:
        return f"attention error max {mx:.3g} mean {mean:.3g}"
    return None


# ------------------------------------------------------------ rounded encodings
# A path that evaluates a value in fp32 and then rounds it to E4M3 or NVFP4
# takes its rounding decisions on a value within delta of the oracle's fp64
# value. Rounding is monotone, so the acceptable bytes are exactly the
# roundings of the interval [x - delta, x + delta]: with delta small against
# the code spacing, the rounding of either end. delta = 0 demands equality.

def check_e4m3_within(got, x, delta):
    """got: E4M3 bytes; x: fp64 values; delta: >= 0, broadcastable to x.
    Returns (message or None, number of elements accepted only through delta)."""
    got = np.asarray(got, dtype=np.uint8)
    x = np.asarray(x, dtype=np.float64)
    delta = np.broadcast_to(np.asarray(delta, dtype=np.float64), x.shape)
    exact = e4m3_encode(x)
    lo, hi = e4m3_encode(x - delta), e4m3_encode(x + delta)
    ok = (got == exact) | (got == lo) | (got == hi)
    if not ok.all():
        i = np.argwhere(~ok)[0]
        return (f"E4M3 byte {got[tuple(i)]:#04x} at {tuple(i)} is no rounding of "
                f"{x[tuple(i)]!r} +- {delta[tuple(i)]:.3g}", 0)
    return None, int(np.count_nonzero(got != exact))


def check_nvfp4_within(codes, scales, x, delta):
    """codes: packed uint8 [..., 64]; scales: row-major uint8 [..., 8]; x: fp64
    [..., 128]; delta: >= 0, broadcastable to x. Each 16-element group's scale
    byte must be the scale of an amax within the deltas of the group's amax,
    and with that scale each code the rounding of a value within delta of x_i
    (either sign where that interval holds 0). Returns (message or None,
    number of groups accepted only through delta)."""
    x = np.asarray(x, dtype=np.float64)
    delta = np.broadcast_to(np.asarray(delta, dtype=np.float64), x.shape)
    g = x.reshape(*x.shape[:-1], -1, GROUP)
    d = delta.reshape(g.shape)
    a = np.abs(g)
    amax, dmax = a.max(axis=-1), d.max(axis=-1)
    sb = np.asarray(scales, dtype=np.int64)
    sb_lo = nearest_even_index(np.maximum(amax - dmax, 0.0), 6.0 * E4M3_MID)
    sb_hi = nearest_even_index(amax + dmax, 6.0 * E4M3_MID)
    sb_exact = nearest_even_index(amax, 6.0 * E4M3_MID)
    bad = (sb < sb_lo) | (sb > sb_hi)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        return f"scale byte {sb[i]} of group {i} outside [{sb_lo[i]}, {sb_hi[i]}]", 0
    s = E4M3_POS[sb][..., None]
    nib = unpack_nibbles(codes).astype(np.int64).reshape(g.shape)
    mag, neg = nib & 7, (nib >> 3) == 1

    def mag_of(v):
        return np.where(s == 0.0, 0, nearest_even_index(v / np.where(s == 0.0, 1.0, s), E2M1_MID))

    m_lo, m_hi = mag_of(np.maximum(a - d, 0.0)), mag_of(a + d)
    ok_mag = (mag >= m_lo) & (mag <= m_hi)
    either_sign = (mag == 0) & (a <= d)
    ok_sign = either_sign | (neg == np.signbit(g))
    ok = ok_mag & ok_sign
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        return (f"code {nib[i]:#x} at {i} is no rounding of {g[i]!r} +- {d[i]:.3g} "
                f"with scale byte {sb[i[:-1]]}", 0)
    exact_mag = mag_of(a)
    differs = (sb != sb_exact) | np.any(mag != np.where(sb[..., None] == sb_exact[..., None],
                                                         exact_mag, mag), axis=-1)
    return None, int(np.count_nonzero(differs))
