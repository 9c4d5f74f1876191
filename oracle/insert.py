"""Cache insertion after the QKV projection (oracle; test infrastructure).

The pages describe a fused path from the QKV projection through
normalisation and RoPE to the cache insert, which avoids writing the full
intermediate tensor to HBM and reading it back (MiniMax-M3.1-Flash serving
summary, section "Reduce both data movement and resource waits"). The
projection itself needs model weights; this oracle covers everything after
it, for the new tokens of one layer.

Input: the projection output, bf16, one row per new token, heads of 128
channels laid out as
    [q: Hq heads][q_idx: Hq_idx heads][k: Hkv heads][v: Hkv heads][k_idx: Hidx heads]
with Hq = 8 Hkv and Hq_idx = 8 Hidx (8 query heads per key head, as in the
decode path).

Per token t at position pos[t]:
  1. RMSNorm per head, optional: y = x / sqrt(mean_c(x_c^2) + eps) * w_c, with
     one weight vector for the query heads (q and q_idx) and one for the key
     heads (k and k_idx); V is not normalised.
  2. RoPE in the rotate-half form on the first r = rotary_dim channels of the
     q, q_idx, k and k_idx heads: for i < r/2, with
     angle_i = pos * theta^(-2i/r),
        y_i       = x_i cos(angle_i) - x_{i+r/2} sin(angle_i)
        y_{i+r/2} = x_{i+r/2} cos(angle_i) + x_i sin(angle_i);
     channels r .. 127 are unchanged. V is not rotated.
  3. k, v and k_idx are quantised to NVFP4 and stored at slot slot_mapping[t]
     of their pools (nvfp4.write_cache; slot < 0: not stored).
  4. q and q_idx are rounded to FP8 E4M3 (nearest, ties to even, satfinite):
     the FP8 queries of the decode step.
Steps 1-2 are evaluated in fp64. The NVFP4 writer takes fp32 sources, so the
fp64 values are rounded to fp32 before step 3; step 4 rounds the fp64 value.

Pins: tests/test_oracle_insert.py (bf16 decoding against torch's bfloat16;
RMSNorm's unit RMS and scale invariance; RoPE at position 0 and with r = 0,
the rotation of a unit vector against cos/sin of the closed-form angle,
pair norms, relative-position invariance of dot products; where each segment
of the row lands).
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_encode
from .nvfp4 import write_cache

HEAD_DIM = 128
HEADS_PER_KEY = 8


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: the upper half of an fp32 word."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def rms_norm(x, w, eps: float):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope_angles(pos, rotary_dim: int, theta: float):
    """angle[t, i] = pos[t] * theta^(-2i/r) for i < r/2 (fp64)."""
    pos = np.asarray(pos, dtype=np.float64).reshape(-1)
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * i / rotary_dim)
    return pos[:, None] * inv_freq[None, :]


def rope(x, pos, rotary_dim: int, theta: float):
    """Rotate-half RoPE on the first rotary_dim channels of x [T, H, D] (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    if rotary_dim == 0:
        return x.copy()
    h = rotary_dim // 2
    ang = rope_angles(pos, rotary_dim, theta)[:, None, :]      # [T, 1, h]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :h], x[..., h:rotary_dim]
    y = x.copy()
    y[..., :h] = lo * c - hi * s
    y[..., h:rotary_dim] = hi * c + lo * s
    return y


def split_row(rows, hq: int, hq_idx: int, hkv: int, hidx: int):
    """Projection rows [T, (hq + hq_idx + 2 hkv + hidx) * 128] -> the five
    head tensors [T, heads, 128] in row order (q, q_idx, k, v, k_idx)."""
    rows = np.asarray(rows)
    t = rows.shape[0]
    out, c = [], 0
    for n in (hq, hq_idx, hkv, hkv, hidx):
        out.append(rows[:, c:c + n * HEAD_DIM].reshape(t, n, HEAD_DIM))
        c += n * HEAD_DIM
    assert c == rows.shape[1], "row width does not match the head counts"
    return out


def transform(rows_bf16, pos, hkv: int, hidx: int, q_norm_w=None, k_norm_w=None,
              eps: float = 1e-6, rotary_dim: int = 128, theta: float = 10000.0):
    """Steps 1-2: the fp64 tensors (q, q_idx, k, v, k_idx) before any rounding."""
    hq, hq_idx = HEADS_PER_KEY * hkv, HEADS_PER_KEY * hidx
    x = bf16_to_f64(rows_bf16)
    q, qi, k, v, ki = split_row(x, hq, hq_idx, hkv, hidx)
    if q_norm_w is not None:
        q, qi = rms_norm(q, q_norm_w, eps), rms_norm(qi, q_norm_w, eps)
    if k_norm_w is not None:
        k, ki = rms_norm(k, k_norm_w, eps), rms_norm(ki, k_norm_w, eps)
    q, qi, k, ki = (rope(a, pos, rotary_dim, theta) for a in (q, qi, k, ki))
    return q, qi, k, v.copy(), ki


def insert(rows_bf16, pos, slot_mapping, k_pool, v_pool, idx_pool, q_norm_w=None,
           k_norm_w=None, eps: float = 1e-6, rotary_dim: int = 128, theta: float = 10000.0):
    """Steps 1-4. Pools are (codes, scales) pairs updated in place; returns
    (q_fp8 [T, Hq, 128] uint8, q_idx_fp8 [T, Hq_idx, 128] uint8)."""
    hkv, hidx = k_pool[0].shape[1], idx_pool[0].shape[1]
    q, qi, k, v, ki = transform(rows_bf16, pos, hkv, hidx, q_norm_w, k_norm_w, eps,
                                rotary_dim, theta)
    for (codes, scales), src in ((k_pool, k), (v_pool, v), (idx_pool, ki)):
        write_cache(codes, scales, src.astype(np.float32), slot_mapping)
    return e4m3_encode(q), e4m3_encode(qi)
