"""Seeded synthetic inputs for MSA decode over an NVFP4 paged KV cache.

This package is shared by the CPU oracle's tests and by the HIP path's tests
and benchmark. It holds no arithmetic of the method: it draws fp32 sources,
FP8 queries, head weights, sequence lengths and block tables, and nothing
else. Every draw is a pure function of (seed, stream, element index), so any
page or query can be regenerated on either device, bit for bit.
"""
from .synth import (  # noqa: F401
    STREAM_K, STREAM_V, STREAM_IDX, STREAM_QIDX, STREAM_QATTN, STREAM_W,
    hash_u32, normal_f32, uniform01_f32, page_sources, query_fp8, head_weights,
)
from .configs import CONFIGS, Workload, get_config, tiny_config  # noqa: F401
