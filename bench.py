"""Decode benchmark: indexer + sparse attention over an NVFP4 paged KV cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

One step = one decode step of one layer: msa_indexer_scan (scan the whole
NVFP4 index cache of every sequence and score its blocks), then
msa_sparse_attn_select_decode (select top-16 + recent blocks per query token
and run exact attention over them, in one launch: the last split of each
(query token, KV head) pair merges the splits' partials).
Inputs are synthetic and already resident in HBM (seeded generator, cache
written by msa_nvfp4_quantize) before the timed region starts.

The timed region launches K steps back to back through prepared library
calls (arguments marshalled once); --graph times HIP-graph replays instead. Prints one JSON
line: query tokens/s (value), achieved HBM GB/s of the step, the indexer
kernel against the HBM roofline (HIP events on the launch stream, eager
launches), and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py --insert

benchmarks the cache-insertion path instead (msa_qkv_rope_insert on 16,384
new tokens, against the same transform done as separate passes) and prints
its own JSON line in the same form.

    python bench.py --mono

benchmarks the one-launch decode step for low concurrency (msa_decode_mono:
scan, selection and attention in one kernel) on the 1 x 4,096-token
workload against the two-launch step, with a sweep of small batches, and
prints its own JSON line in the same form.
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
    p.add_argument("--mono", action="store_true",
                   help="benchmark the one-launch decode step (msa_decode_mono) on the "
                        "1 x 4,096-token workload (or --workload), against the "
                        "two-launch step, plus a sweep of small batches; prints its own "
                        "JSON line")
    p.add_argument("--workload", type=int, default=None,
                   help="workload index (0..4); 2 = 8 x 262,144 tokens")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--insert", action="store_true",
                   help="benchmark the cache-insertion path (msa_qkv_rope_insert) on 16,384 "
                        "new tokens instead of the decode step; prints its own JSON line")
    p.add_argument("--graph", action="store_true",
                   help="time HIP-graph replays of the captured step instead of eager launches")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device-to-device copy (the reference kernel "
                        "for scaling HBM byte counters) and exit")
    p.add_argument("--record-traffic", action="store_true",
                   help="write profiles/traffic_indexer_scan_<workload>.json from the four "
                        "rocprofv3 --pmc output folders given below, and exit")
    p.add_argument("--fetch-dir")
    p.add_argument("--write-dir")
    p.add_argument("--copy-fetch-dir")
    p.add_argument("--copy-write-dir")
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


def scan_bytes_per_workgroup(wl):
    """Index bytes one scan workgroup reads: blocks per workgroup (the
    library's rule for the grid bound, mirrored here) x the index heads'
    9 KiB pages, rounded to 16 bytes."""
    qg = (8 * wl.q_per_seq + 15) // 16
    bpw = 3 if (qg == 1 and wl.num_seqs * wl.max_blocks <= 32768) else 8
    min_grid = 1024 if qg >= 4 else 2048
    while bpw > 1 and wl.num_seqs * -(-wl.max_blocks // bpw) < min_grid:
        bpw >>= 1
    return bpw * wl.num_idx_heads * 128 * IDX_BYTES_PER_TOKEN_HEAD // 16 * 16


def traffic_file(workload_name: str) -> str:
    """The committed HBM-counter record of the index scan on a workload."""
    return os.path.join(ROOT, "profiles", f"traffic_indexer_scan_{workload_name}.json")


SCAN_SOURCES = ("indexer.hip", "scan_body.h", "nvfp4_tile.h")
INSERT_SOURCES = ("insert.hip", "nvfp4_encode.h", "nvfp4_tile.h")
INSERT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_qkv_rope_insert_prefill_16k.json")


def kernel_source_digest(sources=SCAN_SOURCES) -> str:
    """sha256 of a kernel's sources (a stored traffic figure is only
    reported while the kernel it was measured on is unchanged)."""
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "nvfp4_kv_cache_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload_name: str, path=None, sources=SCAN_SOURCES):
    """HBM bytes per launch from a committed rocprofv3 counter record, or
    None when there is none for this workload or the kernel changed."""
    try:
        with open(path or traffic_file(workload_name)) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload_name or rec.get("kernel_source_sha256") != kernel_source_digest(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def _counter_means(run_dir: str, counter: str) -> dict:
    """Mean Counter_Value (KiB) per dispatch and dispatch count, by kernel
    name, from the run_counter_collection.csv rocprofv3 --pmc wrote."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    acc = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                k = acc.setdefault(row["Kernel_Name"], [0.0, 0])
                k[0] += float(row["Counter_Value"])
                k[1] += 1
    return {name: (v / n, n) for name, (v, n) in acc.items()}


def record_traffic(args):
    """Write profiles/traffic_indexer_scan_<workload>.json (or, with
    --insert, the cache-insertion record) from four rocprofv3 --pmc runs:
    FETCH_SIZE and WRITE_SIZE of a bench.py run on the workload, and of
    bench.py --copy-calibration (a plain 1 GiB copy, whose known bytes scale
    each counter). The record carries the sha256 of the kernel's sources;
    bench.py reports it only while they are unchanged."""
    import numpy as np
    from msa_workloads import get_config

    fetch = _counter_means(args.fetch_dir, "FETCH_SIZE")
    write = _counter_means(args.write_dir, "WRITE_SIZE")
    cfetch = _counter_means(args.copy_fetch_dir, "FETCH_SIZE")
    cwrite = _counter_means(args.copy_write_dir, "WRITE_SIZE")

    def pick(d, key):
        names = [n for n in d if key in n]
        if len(names) != 1:
            raise SystemExit(f"expected one kernel matching {key!r}, found {names}")
        return d[names[0]], names[0]
    key = "qkv_rope_insert_kernel" if args.insert else "indexer_kernel"
    (f_kib, f_n), kname = pick(fetch, key)
    (w_kib, w_n), _ = pick(write, key)
    (cf_kib, _), _ = pick(cfetch, "copyBuffer")
    (cw_kib, _), _ = pick(cwrite, "copyBuffer")
    n = 1 << 30
    fs, ws = n / 1024 / cf_kib, n / 1024 / cw_kib
    if args.insert:
        name, path, sources = "prefill_insert_16k", INSERT_TRAFFIC_FILE, INSERT_SOURCES
        alg = insert_algorithmic_bytes(INSERT_TOKENS, INSERT_HKV, INSERT_HIDX)
    else:
        wl = get_config(args.workload)
        name, path, sources = wl.name, traffic_file(wl.name), SCAN_SOURCES
        ids = np.zeros((wl.num_q_tokens, wl.topk + 1), dtype=np.int32)
        # a page mapped by several sequences (a shared prefix) is read once
        nblk = sum(wl.blocks_of(b) for b in range(wl.num_seqs))
        dedup = len(wl.pages_in_use()) < nblk
        alg = algorithmic_bytes(wl, ids, dedup=dedup)[0]
    hbm = int(round(f_kib * 1024 * fs + w_kib * 1024 * ws))
    rec = {"workload": name, "kernel": kname,
           "kernel_source_sha256": kernel_source_digest(sources),
           "fetch_kib_per_dispatch": round(f_kib, 3), "write_kib_per_dispatch": round(w_kib, 3),
           "dispatches": [f_n, w_n], "copy_fetch_kib_per_dispatch": round(cf_kib, 3),
           "copy_write_kib_per_dispatch": round(cw_kib, 3), "copy_bytes_read": n,
           "copy_bytes_written": n, "fetch_scale": round(fs, 5), "write_scale": round(ws, 5),
           "hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": int(alg),
           "traffic_over_algorithmic": round(hbm / alg, 4)}
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


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


# The cache-insertion benchmark: 16,384 new tokens (8 sequences x the last
# 2,048 positions of a 256K context), 4 KV heads and 4 index-key heads, so a
# projection row holds 32 + 32 query heads and 4 + 4 + 4 key/value heads.
INSERT_TOKENS, INSERT_HKV, INSERT_HIDX = 16384, 4, 4
# tokens of the launch the CPU oracle is timed on: all of them (about 7 s of
# CPU work on 16 cores)
INSERT_CPU_SAMPLE = 16384


# tokens per workgroup of the insertion kernel (its launch geometry)
INSERT_TOKENS_PER_WORKGROUP = 2


def insert_read_write_bytes(t, hkv, hidx):
    """Bytes the insertion must read (the bf16 projection rows, positions and
    slots, the two norm weight vectors) and write (the NVFP4 K / V / index
    rows and the FP8 queries)."""
    rows = 8 * hkv + 8 * hidx + 2 * hkv + hidx
    read = t * rows * 128 * 2 + t * (4 + 8) + 2 * 128 * 4
    write = t * (2 * hkv + hidx) * IDX_BYTES_PER_TOKEN_HEAD + t * 8 * (hkv + hidx) * 128
    return read, write


def insert_algorithmic_bytes(t, hkv, hidx):
    """Bytes the insertion must move (read + written)."""
    return sum(insert_read_write_bytes(t, hkv, hidx))


def insert_cpu_baseline(rows, pos, qn, kn, sample):
    """The oracle (as is) on the first `sample` tokens, scaled to tokens/s."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import insert as oins
    from oracle import nvfp4

    cores = len(os.sched_getaffinity(0))
    bits = rows[:sample].cpu().view(__import__("torch").int16).numpy().view(np.uint16)
    pools = [nvfp4.empty_pool(sample // 128 + 1, h) for h in (INSERT_HKV, INSERT_HKV, INSERT_HIDX)]
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        oins.insert(bits, pos[:sample], np.arange(sample), *pools, qn, kn, 1e-6, 128, 1e4)
        dt = time.perf_counter() - t0
    return {"value": round(sample / dt, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the first {sample} of {INSERT_TOKENS} tokens through oracle.insert "
                      f"(fp64 RMSNorm and RoPE, NVFP4 and E4M3 encoding); measured {dt:.1f} s"}


def insert_bench(args):
    """One launch of msa_qkv_rope_insert per step over INSERT_TOKENS tokens."""
    import numpy as np
    import torch
    import nvfp4_kv_cache_amd as nb
    from msa_workloads import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    nb.lib()
    t, hkv, hidx = INSERT_TOKENS, INSERT_HKV, INSERT_HIDX
    width = (8 * hkv + 8 * hidx + 2 * hkv + hidx) * 128
    dev = "cuda"
    rows = synth.projection_rows(11, t, width, device=dev)
    pos_np = np.tile(np.arange(262144 - 2048, 262144), t // 2048)
    pos = torch.as_tensor(pos_np, dtype=torch.int32, device=dev)
    slots = torch.arange(t, dtype=torch.int64, device=dev)
    pools = [nb.empty_pool(t // 128, h) for h in (hkv, hkv, hidx)]
    q = torch.empty((t, 8 * hkv, 128), dtype=torch.uint8, device=dev)
    qi = torch.empty((t, 8 * hidx, 128), dtype=torch.uint8, device=dev)
    qn, kn = synth.norm_weights(5, 0).to(dev), synth.norm_weights(5, 1).to(dev)
    fused = nb.msa_qkv_rope_insert(rows, pos, slots, *pools, q, qi, q_norm_w=qn, k_norm_w=kn,
                                   rms_eps=1e-6, rotary_dim=128, rope_theta=1e4, prepare=True)

    # the unfused comparison: the same transform as separate passes that write
    # and re-read the fp32 intermediate (torch elementwise ops for RMSNorm,
    # RoPE and the FP8 query cast; msa_nvfp4_quantize for the three caches).
    # cos/sin are precomputed once (fp64 angles), as a rotary cache would be.
    ang = (torch.as_tensor(pos_np, dtype=torch.float64)[:, None] *
           1e4 ** (-2.0 * torch.arange(64, dtype=torch.float64) / 128))
    cos = ang.cos().float().to(dev)[:, None, :]
    sin = ang.sin().float().to(dev)[:, None, :]
    heads = [8 * hkv, 8 * hidx, hkv, hkv, hidx]

    def unfused():
        x = rows.float().view(t, sum(heads), 128)
        xq, xqi, xk, xv, xki = x.split(heads, dim=1)

        def norm(a, w):
            return a * torch.rsqrt(a.pow(2).mean(-1, keepdim=True) + 1e-6) * w

        def rope(a):
            lo, hi = a[..., :64], a[..., 64:]
            return torch.cat([lo * cos - hi * sin, hi * cos + lo * sin], dim=-1)

        outs = [rope(norm(xq, qn)), rope(norm(xqi, qn)), rope(norm(xk, kn)), xv.contiguous(),
                rope(norm(xki, kn))]
        for (c, sc), src in zip(pools, outs[2:]):
            nb.msa_nvfp4_quantize(src.contiguous(), slots, c, sc)
        q.copy_(outs[0].clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8))
        qi.copy_(outs[1].clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8))

    stream = torch.cuda.current_stream()

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    print(f"[bench] insert: {t} tokens, warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        fused()
    t_w = time.perf_counter()
    warmup_run = args.warmup
    while (time.perf_counter() - t_w) * 1e3 < args.settle_ms:
        for _ in range(10):
            fused()
        warmup_run += 10
        torch.cuda.synchronize()
    # Timed region: cold launches. Before each, a 512 MiB read (a torch sum,
    # ordinary loads) evicts the previous launch's rows and outputs from the
    # L2 and last-level caches and leaves them holding clean lines; a short
    # spin kernel keeps the host's launch latency out; neither is inside the
    # event pair. Each launch then reads its rows from HBM. (An overwrite
    # instead leaves up to the last-level cache's size of dirty lines, whose
    # write-back then lands inside the next launch: reported beside it as
    # launch_us_after_fill.)
    evict = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    fill = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    n_cold = max(args.steps, 100)

    def cold(fn, n, dirty=False):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for i, (e0, e1) in enumerate(ev):
            if dirty:
                fill.fill_(i & 0xFF)
            else:
                evict.sum()
            torch.cuda._sleep(100_000)
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return np.array([e0.elapsed_time(e1) for e0, e1 in ev]) * 1e3

    print(f"[bench] insert: timed region: {n_cold} cold launches", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cold_us = cold(fused, n_cold)
    wall = time.perf_counter() - t0
    med = float(np.median(cold_us))
    mean = float(np.mean(cold_us))
    p10, p90 = (float(x) for x in np.percentile(cold_us, [10, 90]))
    after_fill = float(np.median(cold(fused, 50, dirty=True)))
    # secondary: K launches back to back (rows can stay in the caches)
    us_warm = timed(fused, args.steps)
    for _ in range(3):
        unfused()
    us_unfused = timed(unfused, max(3, args.steps // 5))
    alg = insert_algorithmic_bytes(t, hkv, hidx)
    achieved = alg / (mean * 1e-6) / 1e9

    # stream ceiling: a plain kernel that reads and writes the insertion's
    # algorithmic bytes at once (msa_stream_probe: the same read:write mix,
    # no arithmetic), at the insertion's read bytes per workgroup and at
    # 1 MiB; mean of 50 cold launches each (same protocol)
    read_b, write_b = insert_read_write_bytes(t, hkv, hidx)
    src = torch.full((read_b // 16 * 16,), 3, dtype=torch.uint8, device=dev)
    dst = torch.empty((write_b // 16 * 16,), dtype=torch.uint8, device=dev)
    chunks, best = {}, None
    for chunk in (read_b // t * INSERT_TOKENS_PER_WORKGROUP // 16 * 16, 1 << 20):
        probe = nb.msa_stream_probe(src, dst, chunk, prepare=True)
        for _ in range(5):
            probe()
        pus = float(np.mean(cold(probe, 50)))
        gbs = (src.numel() + dst.numel()) / (pus * 1e-6) / 1e9
        chunks[str(chunk)] = {"us": round(pus, 2), "gbs": round(gbs, 1)}
        best = gbs if best is None else max(best, gbs)
    del src, dst, evict, fill
    stream_ceiling = {"kernel": "stream_probe_kernel (msa_stream_probe)", "read_bytes": read_b,
                      "write_bytes": write_b, "chunks": chunks, "best_gbs": round(best, 1),
                      "frac_of_peak": round(best / HBM_PEAK_GBS, 4)}
    res = {
        "metric": "cache-insert tokens/s (bf16 QKV projection rows -> RMSNorm, RoPE, NVFP4 K/V/index pages, FP8 queries)",
        "value": round(t / (med * 1e-6), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warmup_run,
        "ms_per_step": round(med / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) x 2^U{-3..3} per head, bf16; U(0.5,1.5) norm weights)",
        "config": {"workload": "prefill_insert_16k", "tokens": t, "kv_heads": hkv,
                   "index_heads": hidx, "q_heads": 8 * hkv, "index_q_heads": 8 * hidx,
                   "rotary_dim": 128, "rope_theta": 1e4, "rms_norm": True,
                   "positions": "8 x (262,144 - 2,048 .. 262,143)"},
        "timing": (f"median of {n_cold} cold launches (max(steps, 100)), each timed with HIP "
                   f"events after a 512 MiB read that evicts the caches (clean) and a spin kernel, "
                   f"both outside the event pair"),
        "cold_launches_timed": n_cold,
        "timed_region_wall_s": round(wall, 4),
        "launch_us": {"median": round(med, 2), "mean": round(mean, 2), "p10": round(p10, 2),
                      "p90": round(p90, 2)},
        "launch_us_after_fill": round(after_fill, 2),
        "warm_us_per_step": round(us_warm, 2),
        "unfused_us_per_step": round(us_unfused, 2),
        "unfused": "torch elementwise RMSNorm / RoPE / FP8 cast on the fp32 intermediate + 3 x msa_nvfp4_quantize",
        "roofline": {"bound": "hbm", "kernel": "qkv_rope_insert_kernel (msa_qkv_rope_insert)",
                     "duration": "mean of the cold launches",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes": alg,
                     "traffic": measured_traffic("prefill_insert_16k", INSERT_TRAFFIC_FILE,
                                                 INSERT_SOURCES),
                     "stream_ceiling": stream_ceiling,
                     "frac_of_stream_ceiling": round(achieved / stream_ceiling["best_gbs"], 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] insert: cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = insert_cpu_baseline(rows, pos_np, qn.cpu().numpy(), kn.cpu().numpy(),
                                                  INSERT_CPU_SAMPLE)
    print(json.dumps(res), flush=True)


def mono_bench(args):
    """msa_decode_mono (one launch) against msa_indexer_scan +
    msa_sparse_attn_select_decode (the two-launch step) on one workload
    (default: 1 x 4,096 tokens, 1 query token), plus a sweep of small
    batches; same JSON contract as the decode benchmark."""
    import numpy as np
    import torch
    import nvfp4_kv_cache_amd as nb
    from msa_workloads import get_config, synth, tiny_config
    from msa_workloads.device import device_inputs, fill_pools

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    nb.lib()
    scale = 1.0 / math.sqrt(128)
    stream = torch.cuda.current_stream()

    def setup(wl):
        pools = fill_pools(wl, nb, garbage=False)
        inp = device_inputs(wl)
        tq = wl.num_q_tokens
        ic, isc = pools[synth.STREAM_IDX]
        kc, ks = pools[synth.STREAM_K]
        vc, vs = pools[synth.STREAM_V]
        r = dict(wl=wl, pools=pools, inp=inp)
        r["ws_m"] = nb.mono_workspace(wl.num_seqs, wl.q_per_seq, wl.num_q_heads, wl.max_blocks)
        r["ws_i"] = nb.indexer_workspace(wl.num_seqs, wl.q_per_seq, wl.max_blocks)
        r["ws_a"] = nb.attn_workspace(wl.num_seqs, wl.q_per_seq, wl.num_q_heads, wl.topk + 1)
        for k in ("m", "3"):
            r["ids" + k] = torch.empty((tq, wl.topk + 1), dtype=torch.int32, device="cuda")
            r["out" + k] = torch.empty((tq, wl.num_q_heads, 128), dtype=torch.float32,
                                       device="cuda")
        bsc = r["ws_i"][: tq * wl.max_blocks * 4].view(torch.float32).view(tq, wl.max_blocks)
        r["mono"] = nb.msa_decode_mono(ic, isc, inp["q_idx"], inp["w"], kc, ks, vc, vs,
                                       inp["q_attn"], inp["block_table"], inp["seq_lens"],
                                       wl.q_per_seq, scale, r["outm"], r["ws_m"],
                                       out_ids=r["idsm"], prepare=True)
        scan = nb.msa_indexer_scan(ic, isc, inp["q_idx"], inp["w"], inp["block_table"],
                                   inp["seq_lens"], wl.q_per_seq, bsc, prepare=True)
        attn = nb.msa_sparse_attn_select_decode(kc, ks, vc, vs, inp["q_attn"],
                                                inp["block_table"], inp["seq_lens"],
                                                wl.q_per_seq, bsc, scale, r["out3"], r["ws_a"],
                                                out_ids=r["ids3"], prepare=True)

        def three():
            scan()
            attn()
        r["three"] = three
        return r

    def settle(fn, n0):
        t_w = time.perf_counter()
        for _ in range(n0):
            fn()
        torch.cuda.synchronize()
        n = n0
        while (time.perf_counter() - t_w) * 1e3 < args.settle_ms:
            for _ in range(20):
                fn()
            n += 20
            torch.cuda.synchronize()
        return n

    def wall_us(fn, k):
        t0 = time.perf_counter()
        for _ in range(k):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / k * 1e6

    def event_us(fn, k):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(k)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3

    wl = get_config(0 if args.workload is None else args.workload)
    print(f"[bench] mono: workload {wl.name}: filling pools", file=sys.stderr, flush=True)
    r = setup(wl)
    warm = settle(lambda: (r["mono"](), r["three"]()), args.warmup)
    same = (torch.equal(r["idsm"], r["ids3"]) and
            torch.equal(r["outm"].view(torch.int32), r["out3"].view(torch.int32)))
    tq = wl.num_q_tokens
    us_mono = wall_us(r["mono"], args.steps)
    us_three = wall_us(r["three"], args.steps)
    ev_mono = event_us(r["mono"], args.steps)
    ev_three = event_us(r["three"], args.steps)
    ids_np = r["idsm"].cpu().numpy()
    idx_bytes, rest_bytes, union = algorithmic_bytes(wl, ids_np)
    step_bytes = idx_bytes + rest_bytes
    # every block's K/V is read once more than the selection needs (the
    # partials of unselected blocks are computed and dropped)
    kv_read = sum(wl.blocks_of(b) for b in range(wl.num_seqs)) * 2 * wl.num_kv_heads * \
        KV_BYTES_PER_BLOCK_HEAD * wl.q_per_seq

    sweep = []
    for lens, q in [([4096] * 2, 1), ([4096] * 4, 1), ([8192], 1), ([16384], 1),
                    ([4096] * 2, 2), ([4096], 4)]:
        w2 = tiny_config(lens, q, seed=len(lens) * 10 + q, spare_pages=0, permute=False,
                         name=f"{len(lens)}x{lens[0]}_q{q}")
        r2 = setup(w2)
        settle(lambda: (r2["mono"](), r2["three"]()), 5)
        sweep.append({"workload": w2.name, "num_seqs": len(lens), "context_tokens": lens[0],
                      "q_per_seq": q,
                      "mono_us": round(wall_us(r2["mono"], args.steps), 2),
                      "two_launch_us": round(wall_us(r2["three"], args.steps), 2)})
        del r2
    res = {
        "metric": "decode query-tokens/s + achieved HBM GB/s (indexer+sparse-attn, 1 layer)",
        "value": round(tq / (us_mono * 1e-6), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(us_mono * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "launch": "eager (prepared calls), one kernel per step (msa_decode_mono)",
        "data": "synthetic (seeded N(0,1) fp32 sources quantised to NVFP4 on the GPU; "
                "FP8 queries; U(0,1) head weights)",
        "config": {"workload": wl.name, "num_seqs": wl.num_seqs,
                   "context_tokens": int(max(wl.seq_lens)), "q_per_seq": wl.q_per_seq,
                   "kv_heads": wl.num_kv_heads, "index_heads": wl.num_idx_heads,
                   "q_heads": wl.num_q_heads, "head_dim": 128, "block_tokens": 128,
                   "topk": wl.topk},
        "achieved_hbm_gbs": round(step_bytes / (us_mono * 1e-6) / 1e9, 1),
        "hbm_frac_of_peak": round(step_bytes / (us_mono * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": int(step_bytes),
        "kv_bytes_read_per_step": int(kv_read),
        "two_launch_us_per_step": round(us_three, 2),
        "speedup_vs_two_launch": round(us_three / us_mono, 3),
        "bit_identical_to_two_launch": bool(same),
        "kernels_us": {"msa_decode_mono": round(ev_mono, 2),
                       "two_launch_step_events": round(ev_three, 2)},
        "sweep": sweep,
        "roofline": {"bound": "hbm", "kernel": "mono_kernel (msa_decode_mono)",
                     "achieved": round(step_bytes / (ev_mono * 1e-6) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_bytes / (ev_mono * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": int(step_bytes), "traffic": None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_blocks)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.record_traffic:
        if args.workload is None:
            args.workload = 2
        record_traffic(args)
        return
    if args.insert:
        insert_bench(args)
        return
    if args.mono:
        mono_bench(args)
        return
    if args.workload is None:
        args.workload = 2

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
    groups = shared_groups(wl, nb)
    dedup = groups[2] > 0
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
        # attention in one launch (the last split of each pair merges)
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

    stream = torch.cuda.current_stream()

    # Headline (timed region): N = max(K, 100) cold steps. Before each, a
    # 512 MiB buffer is overwritten (more than the 256 MB last-level cache
    # and the L2s hold, so no input of the step is left in a cache) and a
    # short spin kernel keeps the host's launch latency out; neither is
    # inside the event pair. Each step is timed with a pair of HIP events on
    # the launch stream (the library launches on torch's current stream).
    # Reported: the median with p10 / p90. (An event recorded between the
    # two launches of a step costs ~5 us by itself, traced: the stage split
    # is therefore measured in a separate loop below.)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    n_cold = max(args.steps, 100)

    def cold_steps(n, split):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3 if split else 2)]
              for _ in range(n)]
        for i, e in enumerate(ev):
            flush.fill_(i & 0xFF)
            torch.cuda._sleep(100_000)
            e[0].record(stream)
            scan()
            if split:
                e[1].record(stream)
            select_attend()
            e[-1].record(stream)
        torch.cuda.synchronize()
        return ev

    print(f"[bench] timed region: {n_cold} cold steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev = cold_steps(n_cold, False)
    wall = time.perf_counter() - t0
    step_us = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3
    med = float(np.median(step_us))
    p10, p90 = (float(x) for x in np.percentile(step_us, [10, 90]))
    if not (torch.equal(out, eager_out) and torch.equal(ids, eager_ids)):
        raise RuntimeError("cold steps differ from the warm-up step")
    # cold stage split: the scan, then selection + attention (merge included),
    # with the extra event between them
    ev = cold_steps(max(args.steps, 50), True)
    scan_us = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3
    attn_us = np.array([e[1].elapsed_time(e[2]) for e in ev]) * 1e3

    # Secondary: warm steps, K back to back (the selected K/V blocks and the
    # scores can stay in the last-level cache between steps). Eager prepared
    # launches by default; with --graph, HIP-graph replays (g steps per
    # graph, g the largest divisor of K up to 10) after checking one replay
    # bit for bit against the eager step (graph kernel nodes measured ~3 us
    # slower each than stream launches here).
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
        launch = f"hip_graph ({g} steps per replay) for the warm steps"
        tw = time.perf_counter()
        for _ in range(args.steps // g):
            graph.replay()
        torch.cuda.synchronize()
        warm_wall = time.perf_counter() - tw
    else:
        launch = "eager (prepared calls)"
        tw = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        warm_wall = time.perf_counter() - tw
    warm_us = warm_wall / args.steps * 1e6

    # warm per-stage durations (events around each launch, back to back)
    evw = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in evw:
        e[0].record(stream)
        scan()
        e[1].record(stream)
        select_attend()
        e[2].record(stream)
    torch.cuda.synchronize()
    warm_scan = float(np.mean([e[0].elapsed_time(e[1]) for e in evw])) * 1e3
    warm_attn = float(np.mean([e[1].elapsed_time(e[2]) for e in evw])) * 1e3

    # read ceiling: a plain streaming read (msa_read_probe, the scan's loads
    # with no arithmetic) of as many bytes as the scan's index cache, one
    # contiguous chunk per workgroup, at the scan's bytes per workgroup and
    # at 1 MiB; best of 20 launches each (the buffer is larger than every
    # cache, so each launch reads HBM)
    idx_cache_bytes = (ic.numel() + isc.numel()) if not dedup else None
    ceiling = None
    if idx_cache_bytes is not None:
        del flush
        probe_buf = torch.empty(idx_cache_bytes // 16 * 16, dtype=torch.uint8, device=dev)
        probe_buf.fill_(3)
        per_wg = scan_bytes_per_workgroup(wl)
        best = None
        chunks = {}
        for chunk in (per_wg, 1 << 20):
            sink = torch.zeros(-(-probe_buf.numel() // chunk), dtype=torch.int32, device=dev)
            probe = nb.msa_read_probe(probe_buf, chunk, sink, prepare=True)
            for _ in range(5):
                probe()
            pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(20)]
            for e0, e1 in pe:
                e0.record(stream)
                probe()
                e1.record(stream)
            torch.cuda.synchronize()
            us = min(e0.elapsed_time(e1) for e0, e1 in pe) * 1e3
            gbs = probe_buf.numel() / (us * 1e-6) / 1e9
            chunks[str(chunk)] = {"us": round(us, 2), "gbs": round(gbs, 1)}
            best = gbs if best is None else max(best, gbs)
        del probe_buf
        ceiling = {"kernel": "read_probe_kernel (msa_read_probe)", "bytes": idx_cache_bytes,
                   "chunks": chunks, "best_gbs": round(best, 1),
                   "frac_of_peak": round(best / HBM_PEAK_GBS, 4)}

    ids_np = ids.cpu().numpy()
    idx_bytes, attn_bytes, union = algorithmic_bytes(wl, ids_np, dedup=dedup)
    step_bytes = idx_bytes + attn_bytes
    scan_mean = float(np.mean(scan_us))
    idx_gbs = idx_bytes / (scan_mean * 1e-6) / 1e9
    res = {
        "metric": "decode query-tokens/s + achieved HBM GB/s (indexer+sparse-attn, 1 layer)",
        "value": round(tq / (med * 1e-6), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warmup_run,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(med * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "timing": (f"median of {n_cold} cold steps (max(steps, 100)), each timed with HIP events "
                   f"after a 512 MiB overwrite and a spin kernel outside the event pair"),
        "cold_steps_timed": n_cold,
        "timed_region_wall_s": round(wall, 4),
        "step_us": {"median": round(med, 2), "p10": round(p10, 2), "p90": round(p90, 2)},
        "launch": launch,
        "data": "synthetic (seeded N(0,1) fp32 sources quantised to NVFP4 on the GPU; "
                "FP8 queries; U(0,1) head weights)",
        "config": {"workload": wl.name, "num_seqs": wl.num_seqs,
                   "context_tokens": int(max(wl.seq_lens)), "q_per_seq": wl.q_per_seq,
                   "kv_heads": wl.num_kv_heads, "index_heads": wl.num_idx_heads,
                   "q_heads": wl.num_q_heads, "head_dim": 128, "block_tokens": 128,
                   "topk": wl.topk,
                   "shared_prefix_groups": int(len(groups[0])),
                   "shared_prefix_blocks": [int(x) for x in groups[1].cpu().tolist()]},
        "achieved_hbm_gbs": round(step_bytes / (med * 1e-6) / 1e9, 1),
        "hbm_frac_of_peak": round(step_bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": int(step_bytes),
        "kernels_us_cold": {
            "method": "separate cold loop with an event between the two launches (the middle "
                      "event adds its own few us to the second stage)",
            "msa_indexer_scan": {"median": round(float(np.median(scan_us)), 2),
                                 "mean": round(scan_mean, 2)},
            "msa_sparse_attn_select_decode": {"median": round(float(np.median(attn_us)), 2),
                                              "mean": round(float(np.mean(attn_us)), 2)}},
        "warm": {"us_per_step": round(warm_us, 2),
                 "value": round(tq / (warm_us * 1e-6), 1),
                 "hbm_frac_of_peak": round(step_bytes / (warm_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                 "kernels_us": {"msa_indexer_scan": round(warm_scan, 2),
                                "msa_sparse_attn_select_decode": round(warm_attn, 2)},
                 "method": f"{args.steps} back-to-back steps after the settle phase"},
        "selected_blocks_union": int(union),
        "read_ceiling": ceiling,
        "roofline": {"bound": "hbm", "kernel": "indexer_kernel (msa_indexer_scan)",
                     "achieved": round(idx_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(idx_gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": int(idx_bytes),
                     "duration": "mean of the scan's HIP-event durations over the cold steps",
                     "frac_of_read_ceiling": (round(idx_gbs / ceiling["best_gbs"], 4)
                                              if ceiling else None),
                     "traffic": measured_traffic(wl.name)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_blocks)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
