"""Lay a workload's synthetic data into GPU pools through the library's own
cache writer. This module moves data only: the quantiser it calls is the
binding passed in as `nb` (the HIP library), never re-implemented here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import synth

STREAMS = (synth.STREAM_K, synth.STREAM_V, synth.STREAM_IDX)


def page_rows(wl) -> dict:
    """physical page -> number of written rows (the most any sequence uses)."""
    rows = {}
    for b in range(wl.num_seqs):
        L = int(wl.seq_lens[b])
        for j in range(wl.blocks_of(b)):
            p = int(wl.block_table[b, j])
            rows[p] = max(rows.get(p, 0), min(128, L - 128 * j))
    return rows


def fill_pools(wl, nb, device="cuda", garbage=True, chunk_pages=256, overrides=None):
    """Allocate and fill the K, V and index pools of `wl` on the GPU.

    overrides: optional callable(stream, pages_np, src_tensor) -> src_tensor
    applied to each chunk's fp32 sources before quantisation (planted tests).
    Returns dict stream -> (codes, scales).
    """
    rows = page_rows(wl)
    pages = np.array(sorted(rows), dtype=np.int64)
    nrows = np.array([rows[p] for p in pages], dtype=np.int64)
    pools = {}
    for st in STREAMS:
        h = wl.num_heads_of(st)
        codes, scales = nb.empty_pool(wl.num_pages, h, device=device)
        if garbage:
            g = torch.Generator(device=device)
            g.manual_seed(1234 + st)
            codes.copy_(torch.randint(0, 256, codes.shape, dtype=torch.uint8, device=device,
                                      generator=g))
            scales.copy_(torch.randint(0, 256, scales.shape, dtype=torch.uint8, device=device,
                                       generator=g))
        else:
            codes.zero_()
            scales.zero_()
        for c0 in range(0, len(pages), chunk_pages):
            pg = pages[c0:c0 + chunk_pages]
            nr = nrows[c0:c0 + chunk_pages]
            src = wl.sources(st, pg, device=device)
            if overrides is not None:
                src = overrides(st, pg, src)
            r = np.arange(128)
            slots = (pg[:, None] * 128 + r[None, :])
            slots = np.where(r[None, :] < nr[:, None], slots, -1).reshape(-1)
            nb.msa_nvfp4_quantize(src.contiguous(), torch.from_numpy(slots).to(device),
                                  codes, scales)
        pools[st] = (codes, scales)
    return pools


def shared_groups(wl, nb, device="cuda"):
    """The workload's shared-prefix groups as the library derives them from
    a host copy of the block table (nb.msa_shared_prefix_groups): device
    tensors (group_lead, group_blocks), the host int max_group_blocks, and
    the device tensor seq_group."""
    bt = torch.from_numpy(np.ascontiguousarray(wl.block_table, dtype=np.int32))
    lens = torch.tensor(wl.seq_lens, dtype=torch.int32)
    return nb.msa_shared_prefix_groups(bt, lens, wl.q_per_seq, device=device)


def device_inputs(wl, device="cuda"):
    return dict(
        q_idx=wl.q_idx().to(device),
        q_attn=wl.q_attn().to(device),
        w=wl.weights().to(device),
        block_table=torch.from_numpy(np.ascontiguousarray(wl.block_table)).to(device),
        seq_lens=torch.tensor(wl.seq_lens, dtype=torch.int32, device=device),
    )
