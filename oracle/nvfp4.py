"""NVFP4 cache encoding and the paged pool (oracle; test infrastructure).

NVFP4 as used here: each group of 16 consecutive channels of one token and
one head is stored as sixteen E2M1 codes plus one shared E4M3 scale, with no
second-level per-tensor scale. The pages describe NVFP4 only as a 4-bit
floating-point format with block-wise shared scaling factors, close to MXFP4
but different in detail (vLLM Delivers Day-0 Support for MiniMax M3.1 Flash,
section "NVFP4 KV Cache and MoE Weights"); this definition reproduces the
pages' 34,560 cache bytes per token against 61,440 for FP8 (MiniMax-M3.1-Flash
lands in vLLM on day one, first paragraph): 4 KV heads x (K, V) x
(64 code bytes + 8 scale bytes) = 576 B per token per layer, times 60 layers.

Quantisation of one group x[0..15] (fp32):
  amax = max |x_i|
  s    = the E4M3 value nearest to amax / 6 (ties to even, saturating at 448)
  m_i  = the E2M1 magnitude nearest to |x_i| / s (ties to even, saturating at 6);
         0 when s == 0
  code_i = (sign bit of x_i) << 3 | index of m_i
  byte_j = code_{2j} | code_{2j+1} << 4
Both roundings are decided by exact comparisons in fp64: amax against 6x the
E4M3 midpoints, |x_i| against s x the E2M1 midpoints (every product is exact).

Dequantisation to FP8 (the pages convert the NVFP4 cache to FP8 before the
matrix multiply; MiniMax-M3.1-Flash lands in vLLM on day one, third
paragraph): value_i = E4M3_nearest_even_satfinite(E2M1[m_i] * s) with the sign
of code_i applied. The product is exact in fp64.

Pool layout (one pool per cache: K, V, index keys), per page of 128 tokens:
  codes  uint8 [num_pages][H][128 tokens][D/2]
  scales uint8 [num_pages][H][128 tokens][D/16]
A token in slot s lives in page s // 128 at row s % 128.

Pins: tests/test_oracle_nvfp4.py (page byte counts; exhaustive scale x code
round trip; dequant table against torch.float8_e4m3fn; hand-derived ties).
"""
from __future__ import annotations

import numpy as np

from .formats import (E2M1_MAG, E2M1_MID, E4M3_MID, E4M3_POS, e4m3_encode,
                      nearest_even_index, e4m3_decode)

GROUP = 16


# ---------------------------------------------------------------- byte counts
def nvfp4_bytes_per_token_head(head_dim: int = 128) -> int:
    return head_dim // 2 + head_dim // GROUP


def fp8_bytes_per_token_head(head_dim: int = 128) -> int:
    return head_dim


def mxfp4_bytes_per_token_head(head_dim: int = 128) -> int:
    """MXFP4 (32-element groups, one 1-byte E8M0 scale): the rejected reading."""
    return head_dim // 2 + head_dim // 32


def kv_bytes_per_token(num_kv_heads=4, head_dim=128, layers=1, fmt="nvfp4") -> int:
    per = {"nvfp4": nvfp4_bytes_per_token_head, "fp8": fp8_bytes_per_token_head,
           "mxfp4": mxfp4_bytes_per_token_head}[fmt](head_dim)
    return 2 * num_kv_heads * per * layers


# ---------------------------------------------------------------- quantise
def quantize_groups(x):
    """x: float32 array [..., 16k] -> (codes uint8 [..., 16k] nibbles, scales uint8 [..., k])."""
    x = np.asarray(x, dtype=np.float32)
    g = x.reshape(*x.shape[:-1], x.shape[-1] // GROUP, GROUP).astype(np.float64)
    a = np.abs(g)
    amax = a.max(axis=-1)
    sbyte = nearest_even_index(amax, 6.0 * E4M3_MID)              # 0..126
    s = E4M3_POS[sbyte]
    thr = (s[..., None] * E2M1_MID)[..., None, :]                  # [..., k, 1, 7] exact
    below = (a[..., None] > thr).sum(axis=-1)                      # midpoints strictly below |x|
    tie = (a[..., None] == thr).any(axis=-1)                       # |x| on a midpoint
    mag = below + (tie & (below % 2 == 1))                         # tie -> even code
    mag = np.where(s[..., None] == 0.0, 0, mag)
    nib = (np.signbit(g).astype(np.int64) << 3) | mag
    return nib.reshape(x.shape).astype(np.uint8), sbyte.astype(np.uint8)


def pack_nibbles(nib):
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def quantize(x):
    """fp32 [..., D] -> (packed codes uint8 [..., D/2], scales uint8 [..., D/16])."""
    nib, sb = quantize_groups(x)
    return pack_nibbles(nib), sb


# ---------------------------------------------------------------- dequantise
def dequant_fp8(codes, scales):
    """(packed codes [..., D/2], scales [..., D/16]) -> (FP8 bytes [..., D], float64 values)."""
    nib = unpack_nibbles(codes)
    s = e4m3_decode(np.repeat(np.asarray(scales, dtype=np.uint8), GROUP, axis=-1))
    prod = E2M1_MAG[nib & 7] * s                                   # exact
    mag = nearest_even_index(prod, E4M3_MID)
    byte = (mag | ((nib.astype(np.int64) >> 3) << 7)).astype(np.uint8)
    return byte, e4m3_decode(byte)


# ---------------------------------------------------------------- paged pool
def empty_pool(num_pages, num_heads, head_dim=128, block_tokens=128, fill=0):
    codes = np.full((num_pages, num_heads, block_tokens, head_dim // 2), fill, dtype=np.uint8)
    scales = np.full((num_pages, num_heads, block_tokens, head_dim // GROUP), fill, dtype=np.uint8)
    return codes, scales


def write_cache(codes_pool, scales_pool, src, slot_mapping):
    """Quantise src [T, H, D] and store token t at slot slot_mapping[t] (< 0: skip)."""
    bt = codes_pool.shape[2]
    c, s = quantize(src)
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        codes_pool[slot // bt, :, slot % bt] = c[t]
        scales_pool[slot // bt, :, slot % bt] = s[t]


def gather_sequence(codes_pool, scales_pool, block_table_row, length):
    """(codes [L, H, D/2], scales [L, H, D/16]) of tokens 0..length-1 of one sequence."""
    bt = codes_pool.shape[2]
    nb = (length + bt - 1) // bt
    pages = np.asarray(block_table_row[:nb], dtype=np.int64)
    c = codes_pool[pages].transpose(0, 2, 1, 3).reshape(nb * bt, codes_pool.shape[1], -1)
    s = scales_pool[pages].transpose(0, 2, 1, 3).reshape(nb * bt, scales_pool.shape[1], -1)
    return c[:length], s[:length]
