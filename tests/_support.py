"""Shared helpers of the GPU parity tests, the smoke check and the benchmark.

GPU side: fill the three NVFP4 pools of a workload through msa_nvfp4_quantize
(slots past a sequence's length are left unwritten: they keep whatever bytes
the pool held, garbage included) and upload queries, weights, tables.
Oracle side: regenerate the same fp32 sources on the CPU from the seeded
generator and run the oracle on them. No oracle input comes from the GPU.
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from msa_workloads import synth  # noqa: E402
from msa_workloads.device import (  # noqa: E402,F401
    STREAMS, device_inputs, fill_pools, page_rows, shared_groups)


def run_step(nb, wl, pools, inp, ws_idx=None, ws_attn=None, out=None, fused=True):
    """One decode step on the GPU.

    fused=True is the launch sequence bench.py times: msa_indexer_scan (or
    msa_indexer_scan_shared when sequences share leading pages), then
    msa_sparse_attn_select_decode (selection inside the attention launch);
    msa_indexer_select on the same block scores then supplies the selected
    blocks' scores and must reproduce the ids. fused=False runs
    msa_indexer_decode, then msa_sparse_attn_decode on its ids."""
    dev = inp["q_idx"].device
    tq = wl.num_q_tokens
    if ws_idx is None:
        ws_idx = nb.indexer_workspace(wl.num_seqs, wl.q_per_seq, wl.max_blocks, device=dev)
    if ws_attn is None:
        ws_attn = nb.attn_workspace(wl.num_seqs, wl.q_per_seq, wl.num_q_heads, wl.topk + 1,
                                    device=dev)
    if out is None:
        out = dict(ids=torch.empty((tq, wl.topk + 1), dtype=torch.int32, device=dev),
                   scores=torch.empty((tq, wl.topk + 1), dtype=torch.float32, device=dev),
                   o=torch.empty((tq, wl.num_q_heads, 128), dtype=torch.float32, device=dev))
    ic, isc = pools[synth.STREAM_IDX]
    kc, ks = pools[synth.STREAM_K]
    vc, vs = pools[synth.STREAM_V]
    scale = 1.0 / math.sqrt(128)
    if fused:
        bscores = ws_idx[: tq * wl.max_blocks * 4].view(torch.float32).view(tq, wl.max_blocks)
        groups = shared_groups(wl, nb, device=dev)
        if groups[2] > 0:
            nb.msa_indexer_scan_shared(ic, isc, inp["q_idx"], inp["w"], inp["block_table"],
                                       inp["seq_lens"], wl.q_per_seq, *groups, bscores)
        else:
            nb.msa_indexer_scan(ic, isc, inp["q_idx"], inp["w"], inp["block_table"],
                                inp["seq_lens"], wl.q_per_seq, bscores)
        nb.msa_sparse_attn_select_decode(kc, ks, vc, vs, inp["q_attn"], inp["block_table"],
                                         inp["seq_lens"], wl.q_per_seq, bscores, scale, out["o"],
                                         ws_attn, out_ids=out["ids"])
        ids2 = torch.empty_like(out["ids"])
        nb.msa_indexer_select(bscores, inp["seq_lens"], wl.q_per_seq, ids2, out["scores"])
        torch.cuda.synchronize()
        assert torch.equal(ids2, out["ids"]), "selection inside attention differs from select"
        return out
    nb.msa_indexer_decode(ic, isc, inp["q_idx"], inp["w"], inp["block_table"], inp["seq_lens"],
                          wl.q_per_seq, out["ids"], ws_idx, out_scores=out["scores"])
    nb.msa_sparse_attn_decode(kc, ks, vc, vs, inp["q_attn"], inp["block_table"],
                              inp["seq_lens"], wl.q_per_seq, out["ids"], scale, out["o"], ws_attn)
    return out


# ------------------------------------------------------------------ oracle side
def tune_host_malloc():
    """Keep freed heap memory for reuse (large numpy temporaries otherwise
    return to the OS and fault in again on every chunk)."""
    import ctypes
    try:
        libc = ctypes.CDLL("libc.so.6")
        libc.mallopt(-3, 1 << 30)   # M_MMAP_THRESHOLD
        libc.mallopt(-1, 1 << 36)   # M_TRIM_THRESHOLD
    except OSError:
        pass


def fp8_values(u8: torch.Tensor) -> np.ndarray:
    """FP8 E4M3 bytes -> float64 through the oracle's decoder."""
    from oracle import formats
    return formats.e4m3_decode(u8.cpu().numpy())


def _oracle_pages(wl, stream, pages, overrides=None):
    """Oracle FP8 values [len(pages)*128, H, 128] of whole physical pages."""
    from oracle import nvfp4
    src = wl.sources(stream, pages, device="cpu")
    if overrides is not None:
        src = overrides(stream, np.asarray(pages), src)
    c, s = nvfp4.quantize(src.numpy())
    return nvfp4.dequant_fp8(c, s)[1]


def oracle_block_scores(wl, b, overrides=None, chunk_pages=16):
    """Oracle block scores [nb_i] of every query token of sequence b.

    The index cache is regenerated and quantised a chunk of pages at a time;
    token scores are per token and block scores per block, so each chunk's
    blocks come out of oracle.msa unchanged."""
    from oracle import msa
    q = fp8_values(wl.q_idx())
    w = wl.weights().numpy().astype(np.float64)
    poss = wl.positions(b)
    nblk = wl.blocks_of(b)
    pages = wl.block_table[b, :nblk].astype(np.int64)
    out = [np.empty(p // 128 + 1) for p in poss]
    for c0 in range(0, nblk, chunk_pages):
        pg = pages[c0:c0 + chunk_pages]
        kh = _oracle_pages(wl, synth.STREAM_IDX, pg, overrides)
        for i, pos in enumerate(poss):
            if c0 * 128 > pos:
                continue
            local = min((c0 + len(pg)) * 128, pos + 1) - 1 - c0 * 128
            row = b * wl.q_per_seq + i
            bs = msa.block_scores(msa.token_scores(q[row], w[row], kh, local), local)
            out[i][c0:c0 + len(bs)] = bs
    return out


def oracle_kv(wl, b, blocks, overrides=None):
    """Oracle K and V values [L, H, 128] of sequence b, filled on `blocks`
    only (the rest stays zero and is never read by sparse attention)."""
    L = int(wl.seq_lens[b])
    kv = {}
    for st in (synth.STREAM_K, synth.STREAM_V):
        arr = np.zeros((wl.blocks_of(b) * 128, wl.num_kv_heads, 128))
        for blk in sorted(set(int(x) for x in blocks if x >= 0)):
            arr[blk * 128:(blk + 1) * 128] = _oracle_pages(
                wl, st, [int(wl.block_table[b, blk])], overrides)
        kv[st] = arr[:L]
    return kv


def record_attention_error(label, errs):
    """Print (and, when MSA_ATTN_ERROR_LOG names a file, append as a JSON
    line) the attention error a check reached: the largest max-abs and the
    largest mean-abs error over its query tokens, against the 2e-2 / 2e-3
    bars."""
    import json
    if not errs:
        return
    mx = max(e[0] for e in errs)
    mean = max(e[1] for e in errs)
    print(f"[attn-error] {label}: max-abs {mx:.3e} (bar 2e-2), mean-abs {mean:.3e} (bar 2e-3) "
          f"over {len(errs)} query tokens", flush=True)
    path = os.environ.get("MSA_ATTN_ERROR_LOG")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps({"check": label, "query_tokens": len(errs), "max_abs": mx,
                                 "mean_abs": mean}) + "\n")


def check_sequence(wl, b, ids, scores, o, overrides=None, check_scores=True, label=None):
    """Oracle checks of one sequence's query tokens. Returns a list of
    failures; prints the attention error reached (record_attention_error)."""
    from oracle import msa
    from oracle.acceptance import attention_error, check_attention, check_selection
    bscores = oracle_block_scores(wl, b, overrides)
    rows = [b * wl.q_per_seq + i for i in range(wl.q_per_seq)]
    kv = oracle_kv(wl, b, np.concatenate([ids[r] for r in rows]), overrides)
    q_attn = fp8_values(wl.q_attn())
    fails, errs = [], []
    scale = 1.0 / math.sqrt(128)
    for i, pos in enumerate(wl.positions(b)):
        row = rows[i]
        bsc = bscores[i]
        gids = ids[row]
        msg = check_selection(bsc, gids, wl.topk)
        if msg:
            fails.append(f"seq {b} q {i}: ids {msg}")
            continue
        valid = gids >= 0
        if check_scores:
            ref_sc = bsc[gids[valid]]
            got_sc = scores[row][valid].astype(np.float64)
            rel = np.max(np.abs(got_sc - ref_sc) / np.maximum(np.abs(ref_sc), 1e-6))
            if rel > 1e-4:
                fails.append(f"seq {b} q {i}: block scores off by {rel:.3g} rel")
        ref_o = msa.sparse_attention(q_attn[row], kv[synth.STREAM_K], kv[synth.STREAM_V], gids,
                                     pos, scale)
        errs.append(attention_error(o[row], ref_o))
        msg = check_attention(o[row], ref_o)
        if msg:
            fails.append(f"seq {b} q {i}: {msg}")
    record_attention_error(label or f"{wl.name} seq {b}", errs)
    return fails


def check_page_bytes(wl, pools, pages, overrides=None):
    """Bit-exact comparison of the GPU pool bytes of `pages` (written rows
    only) with the oracle's quantisation of the same sources."""
    from oracle import nvfp4
    from nvfp4_kv_cache_amd import scales_rows
    rows = page_rows(wl)
    fails = []
    for st, (codes, scales) in pools.items():
        for p in pages:
            p = int(p)
            n = rows.get(p, 0)
            if n == 0:
                continue
            src = wl.sources(st, [p], device="cpu")
            if overrides is not None:
                src = overrides(st, np.array([p]), src)
            c, s = nvfp4.quantize(src.numpy())          # [128, H, 64], [128, H, 8]
            gc = codes[p].cpu().numpy().transpose(1, 0, 2)[:n]
            gs = scales_rows(scales[p:p + 1])[0].cpu().numpy().transpose(1, 0, 2)[:n]
            if not np.array_equal(gc, c[:n]) or not np.array_equal(gs, s[:n]):
                bad = int(np.sum(gc != c[:n]) + np.sum(gs != s[:n]))
                fails.append(f"stream {st} page {p}: {bad} bytes differ")
    return fails
