"""Decode benchmark: indexer + sparse attention over an NVFP4 paged KV cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

One step = one decode step of one layer: msa_indexer_scan (scan the whole
NVFP4 index cache of every sequence and score its blocks), then
msa_sparse_attn_select_decode (select top-16 + recent blocks per query token
and run exact attention over them, in one launch plus the split merge).
Inputs are synthetic and already resident in HBM (seeded generator, cache
written by msa_nvfp4_quantize) before the timed region starts.

The timed region launches K steps back to back through prepared library
calls (arguments marshalled once); --graph times HIP-graph replays instead. Prints one JSON
line: query tokens/s (value), achieved HBM GB/s of the step, the indexer
kernel against the HBM roofline (HIP events on the launch stream, eager
launches), and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
IDX_BYTES_PER_TOKEN_HEAD = 72   # 64 code bytes + 8 scale bytes
KV_BYTES_PER_BLOCK_HEAD = 128 * 72


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--settle-ms", type=float, default=60.0,
                   help="after the warmup steps, keep running untimed steps until this much "
                        "warm-up time has passed (the GPU's clocks settle under sustained load)")
    p.add_argument("--workload", type=int, default=2,
                   help="workload index (0..4); 2 = 8 x 262,144 tokens")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="time HIP-graph replays of the captured step instead of eager launches")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device-to-device copy (the reference kernel "
                        "for scaling HBM byte counters) and exit")
    p.add_argument("--cpu-blocks", type=int, default=2048,
                   help="index blocks of one sequence the CPU oracle scans (time is scaled "
                        "to the whole context when fewer)")
    return p.parse_args()


def algorithmic_bytes(wl, ids, dedup=False):
    """Bytes the method must move per step (never the dense K/V it skips).
    With dedup (the shared-prefix scan) a physical page shared by several
    sequences counts once, with the most tokens any of them sees.
    Returns (scan, rest of the step, selected-block union)."""
    tq, hq = wl.num_q_tokens, wl.num_q_heads
    nblocks = sum(wl.blocks_of(b) for b in range(wl.num_seqs))
    if dedup:
        seen = {}
        for b in range(wl.num_seqs):
            L = int(wl.seq_lens[b])
            for j in range(wl.blocks_of(b)):
                page = int(wl.block_table[b, j])
                seen[page] = max(seen.get(page, 0), min(128, L - 128 * j))
        index_tokens = sum(seen.values())
    else:
        index_tokens = sum(int(L) for L in wl.seq_lens)
    scan = (index_tokens * wl.num_idx_heads * IDX_BYTES_PER_TOKEN_HEAD
            + tq * hq * 128          # FP8 index queries
            + tq * hq * 4            # head weights
            + nblocks * 4)           # block-table entries
    union = 0
    for b in range(wl.num_seqs):
        rows = ids[b * wl.q_per_seq:(b + 1) * wl.q_per_seq]
        union += len(set(int(x) for x in rows.reshape(-1) if x >= 0))
    rest = (tq * (wl.topk + 1) * 4 * 2   # ids written by the selection, read by attention
            + union * 2 * wl.num_kv_heads * KV_BYTES_PER_BLOCK_HEAD
            + tq * hq * 128             # FP8 attention queries
            + tq * hq * 128 * 4)        # fp32 output
    return scan, rest, union


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_indexer_scan_long_context_8x256k.json")


def kernel_source_digest() -> str:
    """sha256 of the scan kernel's sources (a stored traffic figure is only
    reported while the kernel it was measured on is unchanged)."""
    import hashlib
    h = hashlib.sha256()
    for f in ("indexer.hip", "nvfp4_tile.h"):
        with open(os.path.join(ROOT, "nvfp4_kv_cache_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload_name: str):
    """HBM bytes per scan launch from the committed rocprofv3 counter record,
    or None when there is none for this workload or the kernel changed."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload_name or rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration():
    """A plain copy of known size: 1 GiB read and 1 GiB written per launch."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def cpu_baseline(wl, nblk):
    """The oracle (as is) timed on one query token: its index scan over the
    first `nblk` blocks of sequence 0 (scaled to the full context) plus exact
    attention over 17 blocks. Quantising the sources is setup (untimed)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import _support as S
    from msa_workloads import synth
    from oracle import msa, nvfp4

    S.tune_host_malloc()
    cores = len(os.sched_getaffinity(0))
    b, nb_full = 0, wl.blocks_of(0)
    nblk = min(nblk, nb_full)
    pages = wl.block_table[b, :nblk].astype(np.int64)
    q = S.fp8_values(wl.q_idx())[0]
    qa = S.fp8_values(wl.q_attn())[0]
    w = wl.weights().numpy().astype(np.float64)[0]
    enc = {}
    for st in (synth.STREAM_IDX, synth.STREAM_K, synth.STREAM_V):
        pg = pages if st == synth.STREAM_IDX else pages[:17]
        chunks = []
        for c0 in range(0, len(pg), 16):
            src = wl.sources(st, pg[c0:c0 + 16]).numpy()
            chunks.append(nvfp4.quantize(src))
        enc[st] = chunks
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        bs = []
        for c, s in enc[synth.STREAM_IDX]:
            kh = nvfp4.dequant_fp8(c, s)[1]
            local = kh.shape[0] - 1
            bs.append(msa.block_scores(msa.token_scores(q, w, kh, local), local))
        ids = msa.select_blocks(np.concatenate(bs), wl.topk)
        t_idx = time.perf_counter() - t0
        t0 = time.perf_counter()
        kh = np.concatenate([nvfp4.dequant_fp8(c, s)[1] for c, s in enc[synth.STREAM_K]])
        vh = np.concatenate([nvfp4.dequant_fp8(c, s)[1] for c, s in enc[synth.STREAM_V]])
        sel = np.arange(min(17, nblk))
        msa.sparse_attention(qa, kh, vh, sel, kh.shape[0] - 1, 1 / math.sqrt(128))
        t_attn = time.perf_counter() - t0
    per_token = t_idx * (nb_full / nblk) + t_attn
    return {
        "value": round(1.0 / per_token, 4),
        "unit": "query-tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"1 query token of sequence 0: NumPy fp64 oracle index scan (NVFP4->FP8 "
                   f"dequant, token scores, block max) over the first {nblk} of {nb_full} "
                   f"blocks, time scaled x{nb_full / nblk:g}, then top-16 selection and exact "
                   f"attention over 17 blocks; BLAS threads={cores}, elementwise NumPy "
                   f"single-threaded; measured {t_idx + t_attn:.1f} s"),
        "selected_in_sample": int(len(ids)),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch
    import nvfp4_kv_cache_amd as nb
    from msa_workloads import get_config, synth
    from msa_workloads.device import device_inputs, fill_pools, shared_groups

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    nb.lib()
    wl = get_config(args.workload)
    print(f"[bench] workload {wl.name}: filling pools", file=sys.stderr, flush=True)
    pools = fill_pools(wl, nb, garbage=False)
    inp = device_inputs(wl)
    tq = wl.num_q_tokens
    dev = "cuda"
    ws_i = nb.indexer_workspace(wl.num_seqs, wl.q_per_seq, wl.max_blocks)
    ws_a = nb.attn_workspace(wl.num_seqs, wl.q_per_seq, wl.num_q_heads, wl.topk + 1)
    ids = torch.empty((tq, wl.topk + 1), dtype=torch.int32, device=dev)
    out = torch.empty((tq, wl.num_q_heads, 128), dtype=torch.float32, device=dev)
    ic, isc = pools[synth.STREAM_IDX]
    kc, ks = pools[synth.STREAM_K]
    vc, vs = pools[synth.STREAM_V]
    scale = 1.0 / math.sqrt(128)

    bscores = ws_i[: tq * wl.max_blocks * 4].view(torch.float32).view(tq, wl.max_blocks)

    # each library call validated and marshalled once (binding.Prepared):
    # re-issuing it is one ctypes call, so the host stays far ahead of the GPU.
    # A batch whose sequences share leading pages (a cached common prefix)
    # is scanned with msa_indexer_scan_shared: each shared block is read and
    # dequantised once for all the sequences that share it.
    groups = shared_groups(wl)
    dedup = groups[3] > 0
    if dedup:
        scan = nb.msa_indexer_scan_shared(ic, isc, inp["q_idx"], inp["w"], inp["block_table"],
                                          inp["seq_lens"], wl.q_per_seq, *groups, bscores,
                                          prepare=True)
    else:
        scan = nb.msa_indexer_scan(ic, isc, inp["q_idx"], inp["w"], inp["block_table"],
                                   inp["seq_lens"], wl.q_per_seq, bscores, prepare=True)
    select_attend = nb.msa_sparse_attn_select_decode(
        kc, ks, vc, vs, inp["q_attn"], inp["block_table"], inp["seq_lens"], wl.q_per_seq,
        bscores, scale, out, ws_a, out_ids=ids, prepare=True)

    def step():
        # the whole hot path: index scan (scores), then selection + sparse
        # attention in one launch (plus the split merge)
        scan()
        select_attend()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    t_w = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # settle: more untimed steps until settle_ms of warm-up have passed.
    # Measured on MI355X: the first ~100 steps after a short warm-up run ~8%
    # slower (112.7 us vs 103.5 us per step at 8 x 256K) while the clocks
    # ramp up under the sustained HBM load; later loops are steady.
    warmup_run = args.warmup
    while (time.perf_counter() - t_w) * 1e3 < args.settle_ms:
        for _ in range(20):
            step()
        warmup_run += 20
        torch.cuda.synchronize()
    eager_out, eager_ids = out.clone(), ids.clone()

    # timed region: K back-to-back steps, synchronised on both sides. By
    # default the steps are launched eagerly (prepared calls). With --graph
    # they are captured in a HIP graph (g steps per graph, g the largest
    # divisor of K up to 10) and replayed K/g times, after checking one
    # replay bit for bit against the eager step; graph kernel nodes measured
    # ~3 us slower each than stream launches here, so eager is the default.
    if args.graph:
        g = max(d for d in range(1, 11) if args.steps % d == 0)
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            if dedup:
                g_scan = nb.msa_indexer_scan_shared(ic, isc, inp["q_idx"], inp["w"],
                                                    inp["block_table"], inp["seq_lens"],
                                                    wl.q_per_seq, *groups, bscores, prepare=True)
            else:
                g_scan = nb.msa_indexer_scan(ic, isc, inp["q_idx"], inp["w"], inp["block_table"],
                                             inp["seq_lens"], wl.q_per_seq, bscores, prepare=True)
            g_attn = nb.msa_sparse_attn_select_decode(
                kc, ks, vc, vs, inp["q_attn"], inp["block_table"], inp["seq_lens"],
                wl.q_per_seq, bscores, scale, out, ws_a, out_ids=ids, prepare=True)
            g_scan()
            g_attn()
            cap.synchronize()
            with torch.cuda.graph(graph, stream=cap):
                for _ in range(g):
                    g_scan()
                    g_attn()
        torch.cuda.current_stream().wait_stream(cap)
        out.zero_()
        ids.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not (torch.equal(out, eager_out) and torch.equal(ids, eager_ids)):
            raise RuntimeError("graph replay differs from the eager step")
        launch = f"hip_graph ({g} steps per replay)"
        t0 = time.perf_counter()
        for _ in range(args.steps // g):
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        launch = "eager (prepared calls)"
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0

    # per-stage durations with HIP events on the launch stream (the library
    # launches on torch's current stream): the scan, then selection + attention
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in ev:
        e[0].record(stream)
        scan()
        e[1].record(stream)
        select_attend()
        e[2].record(stream)
    torch.cuda.synchronize()
    t_idx = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    t_attn = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3

    # cache effect: the timed steps re-read the same selected K/V blocks, which
    # can stay in the 256 MB last-level cache between steps; a decode across
    # many layers would have evicted them. Median of eager steps timed with
    # events, without and with a 512 MiB overwrite before each step; a short
    # spin kernel ahead of the start event keeps the host's launch latency
    # out of both.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def eager_step_us(cold):
        ts = []
        for _ in range(11):
            if cold:
                flush.fill_(1)
            torch.cuda._sleep(200_000)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))
    warm_us, cold_us = eager_step_us(False), eager_step_us(True)
    del flush

    ids_np = ids.cpu().numpy()
    idx_bytes, attn_bytes, union = algorithmic_bytes(wl, ids_np, dedup=dedup)
    ms = wall / args.steps * 1e3
    step_bytes = idx_bytes + attn_bytes
    idx_gbs = idx_bytes / t_idx / 1e9
    res = {
        "metric": "decode query-tokens/s + achieved HBM GB/s (indexer+sparse-attn, 1 layer)",
        "value": round(tq * args.steps / wall, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warmup_run,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "launch": launch,
        "data": "synthetic (seeded N(0,1) fp32 sources quantised to NVFP4 on the GPU; "
                "FP8 queries; U(0,1) head weights)",
        "config": {"workload": wl.name, "num_seqs": wl.num_seqs,
                   "context_tokens": int(max(wl.seq_lens)), "q_per_seq": wl.q_per_seq,
                   "kv_heads": wl.num_kv_heads, "index_heads": wl.num_idx_heads,
                   "q_heads": wl.num_q_heads, "head_dim": 128, "block_tokens": 128,
                   "topk": wl.topk,
                   "shared_prefix_groups": int(len(groups[2])),
                   "shared_prefix_blocks": [int(x) for x in groups[2].cpu().tolist()]},
        "achieved_hbm_gbs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac_of_peak": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": int(step_bytes),
        "kernels_us": {"msa_indexer_scan": round(t_idx * 1e6, 2),
                       "msa_sparse_attn_select_decode": round(t_attn * 1e6, 2)},
        "selected_blocks_union": int(union),
        "cache_effect": {"method": "median of 11 eager steps timed with HIP events "
                                   "behind a spin kernel",
                         "warm_us": round(warm_us, 2), "cold_us": round(cold_us, 2),
                         "flush_bytes_before_cold_step": 512 << 20},
        "roofline": {"bound": "hbm", "kernel": "indexer_kernel (msa_indexer_scan)",
                     "achieved": round(idx_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(idx_gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": int(idx_bytes),
                     "traffic": measured_traffic(wl.name)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_blocks)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
