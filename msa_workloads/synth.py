"""Counter-based synthetic value generator (torch integer ops; CPU or GPU).

Hash: two rounds of the MurmurHash3 32-bit finaliser ("fmix32", Austin
Appleby, public domain) over a 64-bit element counter mixed with keys derived
from (seed, stream). Integer ops on int64 tensors are exact on every device,
so the CPU and the GPU produce identical words.

Normal variates: the top 16 bits of the hash index a table of the 65,536
midpoint quantiles of N(0,1), Phi^-1((i + 0.5) / 65536), stored as fp32.
This is a 16-bit inverse-CDF discretisation of N(0,1) (|x| <= 4.33); the
table lookup is exact on both devices, unlike log/cos-based transforms whose
last bit differs between CPU and GPU libraries.

Uniform variates: ((h >> 8) + 0.5) * 2^-24, exactly representable in fp32,
strictly inside (0, 1).
"""
from __future__ import annotations

from statistics import NormalDist

import numpy as np
import torch

M32 = 0xFFFFFFFF

# stream ids: one per kind of synthetic tensor
STREAM_K = 0
STREAM_V = 1
STREAM_IDX = 2
STREAM_QIDX = 3
STREAM_QATTN = 4
STREAM_W = 5
STREAM_FILL = 6      # garbage written into never-used page slots by tests
STREAM_PROJ = 7      # QKV projection rows (cache-insertion path)
STREAM_NORMW = 8     # RMSNorm weights (cache-insertion path)

_TABLE_CACHE: dict = {}


def _fmix32_int(x: int) -> int:
    x &= M32
    x ^= x >> 16
    x = (x * 0x85EBCA6B) & M32
    x ^= x >> 13
    x = (x * 0xC2B2AE35) & M32
    x ^= x >> 16
    return x


def _fmix32(x: torch.Tensor) -> torch.Tensor:
    # x: int64 tensor with values in [0, 2^32). Products wrap in int64 two's
    # complement; masking keeps the exact low 32 bits.
    x = x ^ (x >> 16)
    x = (x * 0x85EBCA6B) & M32
    x = x ^ (x >> 13)
    x = (x * 0xC2B2AE35) & M32
    x = x ^ (x >> 16)
    return x


def _keys(seed: int, stream: int) -> tuple[int, int]:
    k1 = _fmix32_int(_fmix32_int(seed * 0x9E3779B1 + 0x7F4A7C15) ^ (stream * 0x85EBCA77))
    k2 = _fmix32_int(k1 ^ 0xC2B2AE3D ^ (stream << 8))
    return k1, k2


def hash_u32(seed: int, stream: int, counter: torch.Tensor) -> torch.Tensor:
    """32-bit hash of int64 counters (values returned as int64 in [0, 2^32))."""
    k1, k2 = _keys(seed, stream)
    counter = counter.to(torch.int64)
    lo = counter & M32
    hi = (counter >> 32) & M32
    h = _fmix32(lo ^ k1)
    h = _fmix32(h ^ ((hi * 0x9E3779B1) & M32) ^ k2)
    return h


def _normal_table(device) -> torch.Tensor:
    key = str(device)
    t = _TABLE_CACHE.get(key)
    if t is None:
        nd = NormalDist()
        vals = np.array([nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)],
                        dtype=np.float64).astype(np.float32)
        t = torch.from_numpy(vals).to(device)
        _TABLE_CACHE[key] = t
    return t


def normal_f32(seed: int, stream: int, counter: torch.Tensor) -> torch.Tensor:
    h = hash_u32(seed, stream, counter)
    return _normal_table(counter.device)[h >> 16]


def uniform01_f32(seed: int, stream: int, counter: torch.Tensor) -> torch.Tensor:
    h = hash_u32(seed, stream, counter)
    return ((h >> 8).to(torch.float32) + 0.5) * (2.0 ** -24)


def page_sources(seed: int, stream: int, pages: torch.Tensor, num_heads: int,
                 head_dim: int = 128, block_tokens: int = 128,
                 outlier_channels: torch.Tensor | None = None,
                 outlier_factor: float = 8.0) -> torch.Tensor:
    """fp32 sources for whole physical pages: [n_pages * block_tokens, H, D].

    Element (page p, token-in-page t, head h, channel d) uses counter
    ((p * block_tokens + t) * H + h) * D + d, so a page's values depend only
    on its physical id (a shared-prefix page is one set of values).
    outlier_channels: optional bool [H, D]; those channels are multiplied by
    outlier_factor (a power of two, so the product is exact).
    """
    dev = pages.device
    per_page = block_tokens * num_heads * head_dim
    base = pages.to(torch.int64).reshape(-1, 1) * per_page
    ctr = base + torch.arange(per_page, device=dev, dtype=torch.int64).reshape(1, -1)
    x = normal_f32(seed, stream, ctr).reshape(-1, num_heads, head_dim)
    if outlier_channels is not None:
        f = torch.where(outlier_channels.to(dev), torch.tensor(outlier_factor, device=dev),
                        torch.tensor(1.0, device=dev)).to(torch.float32)
        x = x * f.reshape(1, num_heads, head_dim)
    return x


def query_fp8(seed: int, stream: int, num_q_tokens: int, num_heads: int,
              head_dim: int = 128) -> torch.Tensor:
    """FP8 E4M3 query bytes [T_q, Hq, D] (uint8, CPU): N(0,1) draws rounded by
    torch's float8_e4m3fn cast (round-to-nearest-even)."""
    n = num_q_tokens * num_heads * head_dim
    x = normal_f32(seed, stream, torch.arange(n, dtype=torch.int64))
    return x.reshape(num_q_tokens, num_heads, head_dim).to(torch.float8_e4m3fn).view(torch.uint8)


def head_weights(seed: int, num_q_tokens: int, num_heads: int) -> torch.Tensor:
    """Indexer head weights U(0,1), fp32 [T_q, Hq] (CPU)."""
    n = num_q_tokens * num_heads
    return uniform01_f32(seed, STREAM_W, torch.arange(n, dtype=torch.int64)).reshape(
        num_q_tokens, num_heads)


def projection_rows(seed: int, num_tokens: int, width: int, device="cpu") -> torch.Tensor:
    """bf16 projection rows [T, width]: N(0,1) draws times a per-(token, head)
    magnitude 2^e, e uniform in -3..3 (exact), rounded to bf16 by torch's
    cast (nearest even). Heads are 128 channels wide."""
    n = num_tokens * width
    x = normal_f32(seed, STREAM_PROJ, torch.arange(n, dtype=torch.int64, device=device))
    heads = torch.arange(n, dtype=torch.int64, device=device) // 128
    e = (hash_u32(seed, STREAM_PROJ + 100, heads) % 7).to(torch.float32) - 3.0
    return (x * torch.exp2(e)).reshape(num_tokens, width).to(torch.bfloat16)


def norm_weights(seed: int, which: int, device="cpu") -> torch.Tensor:
    """RMSNorm weights fp32 [128], U(0.5, 1.5) (which: 0 queries, 1 keys)."""
    u = uniform01_f32(seed, STREAM_NORMW, torch.arange(128, dtype=torch.int64, device=device) + 128 * which)
    return u + 0.5
