"""Element formats, written from their definitions (oracle; test infrastructure).

E4M3 here is the OCP 8-bit floating-point "E4M3FN" encoding: 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits, subnormals when the exponent
field is 0, no infinities, and S.1111.111 as the only NaN pattern, so the
largest finite magnitude is 448. It is both the FP8 type of the queries and
of the dequantised cache (MiniMax-M3.1-Flash lands in vLLM on day one, third
paragraph: the query stays FP8 and the cache is converted to FP8 before the
matrix multiply) and the type of the NVFP4 block scale.

E2M1 is the 4-bit element type of NVFP4: 1 sign bit, 2 exponent bits (bias 1),
1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.

Rounding is "nearest, ties to the even code": the value sets are sorted by
code, so the even code is the one whose mantissa LSB is 0. Values beyond the
largest magnitude saturate to it (satfinite).

Pins: tests/test_oracle_formats.py checks e4m3_decode on all 256 bytes and
e4m3_encode on random values, on every midpoint and just beside it against
torch.float8_e4m3fn casts (an independent library routine), and the E2M1
tables against the format definition.
"""
from __future__ import annotations

import numpy as np


def e4m3_decode(b) -> np.ndarray:
    """E4M3 byte(s) -> float64 value(s). NaN for 0x7F and 0xFF."""
    b = np.asarray(b).astype(np.int64) & 0xFF
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (b & 0x7 == 7), np.nan, mag)
    return sign * mag


# the 127 finite non-negative E4M3 values, indexed by their byte 0x00..0x7E
E4M3_POS = e4m3_decode(np.arange(0x7F))
# midpoints between neighbours: exact in fp64 (at most 5 significant bits)
E4M3_MID = (E4M3_POS[:-1] + E4M3_POS[1:]) / 2.0
E4M3_MAX = 448.0

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MID = (E2M1_MAG[:-1] + E2M1_MAG[1:]) / 2.0   # .25 .75 1.25 1.75 2.5 3.5 5


def nearest_even_index(a, thresholds) -> np.ndarray:
    """Index of the value nearest to a in a sorted value set, given the exact
    midpoints `thresholds` between consecutive values; a tie (a equal to a
    midpoint) goes to the even index; beyond the last midpoint -> last index.

    `a` and `thresholds` must be exact (the comparisons are the whole rule).
    """
    a = np.asarray(a, dtype=np.float64)
    thresholds = np.asarray(thresholds, dtype=np.float64)
    i = np.searchsorted(thresholds, a, side="left")        # count of mids < a
    j = np.minimum(i, len(thresholds) - 1)
    tie = (i < len(thresholds)) & (a == thresholds[j])
    return np.where(tie & (i % 2 == 1), i + 1, i)


def e4m3_encode(x) -> np.ndarray:
    """Finite float64 value(s) -> E4M3 byte(s): nearest, ties to even, satfinite,
    sign kept (so a value that rounds to zero keeps its sign bit)."""
    x = np.asarray(x, dtype=np.float64)
    mag = nearest_even_index(np.abs(x), E4M3_MID)
    return (mag | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)
