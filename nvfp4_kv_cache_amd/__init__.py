"""MI355X-native MiniMax-style sparse-attention decode over an NVFP4 paged KV cache.

The compute lives in libmsa_nvfp4.so (HIP, gfx950; C ABI in include/msa_nvfp4.h).
This package is its thin ctypes binding; PyTorch supplies device memory and
the current HIP stream only.
"""
from .binding import (  # noqa: F401
    LIB_PATH, NOALLOC_MAX_SCORES, MonoPrepared, MsaError, PoolDesc, Prepared, attn_workspace,
    empty_pool, indexer_workspace, lib, mono_block_scores, mono_check, mono_workspace,
    msa_attn_workspace_bytes, msa_decode_mono, msa_decode_mono_workspace_bytes,
    msa_indexer_decode, msa_indexer_decode_noalloc, msa_indexer_scan, msa_indexer_scan_shared,
    msa_indexer_select, msa_indexer_workspace_bytes, msa_shared_prefix_groups, msa_nvfp4_quantize, msa_qkv_rope_insert, msa_read_probe, msa_stream_probe,
    msa_sparse_attn_decode, msa_sparse_attn_select_decode, msa_status_string, pool_desc,
    scales_rows,
)
