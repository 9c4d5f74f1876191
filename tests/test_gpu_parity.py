"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bytes of the cache writer must match bit for bit; selected ids must pass the
acceptance rule (exact unless the oracle's 16th/17th gap is below 1e-4
relative); attention must be within max-abs 2e-2 / mean-abs 2e-3 of the
oracle evaluated in fp64 on the GPU's ids with identical FP8 operands.
"""
import math

import numpy as np
import pytest
import torch

import _support as S
from msa_workloads import get_config, synth, tiny_config
from oracle import formats, nvfp4

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def nb():
    import nvfp4_kv_cache_amd as m
    m.lib()
    return m


def _to_np(out):
    torch.cuda.synchronize()
    return out["ids"].cpu().numpy(), out["scores"].cpu().numpy(), out["o"].cpu().numpy()


def _structural(wl, ids):
    """Properties of the ids that hold at any size, for every query token."""
    for b in range(wl.num_seqs):
        for i, pos in enumerate(wl.positions(b)):
            r = ids[b * wl.q_per_seq + i]
            nbk = pos // 128 + 1
            if nbk <= wl.topk + 1:
                assert r.tolist() == list(range(nbk)) + [-1] * (wl.topk + 1 - nbk), (b, i, r)
            else:
                assert np.all(np.diff(r) > 0) and r[-1] == nbk - 1 and r[0] >= 0, (b, i, r)


# ------------------------------------------------------------------ cache writer
def _special_groups():
    """fp32 rows [T, 4, 128] with rounding ties, saturation, zeros and -0."""
    rng = np.random.default_rng(77)
    x = rng.standard_normal((96, 4, 128)).astype(np.float32)
    g = x.reshape(-1, 16)
    n = g.shape[0]
    for i in range(0, min(n, 126 * 3), 3):              # scale ties and neighbours
        k = (i // 3) % 125
        t = np.float32(6.0 * formats.E4M3_MID[k])
        g[i] = 0
        g[i, i % 16] = t
        g[i + 1] = 0
        g[i + 1, 0] = np.nextafter(t, np.float32(np.inf))
        g[i + 2] = 0
        g[i + 2, 5] = -np.nextafter(t, np.float32(0))
    s = np.float32(1.0)
    g[400] = np.array([6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, -1.25, -1.75,
                       -2.5, -3.5, -5, -0.0], dtype=np.float32) * s
    g[401] = 0.0
    g[402] = -0.0
    g[403] = np.float32(3000.0)
    g[403, 1::2] = -np.float32(2999.0)
    g[404] = np.float32(-6.0 * 2.0 ** -10)
    g[405, :] = np.float32(1e-30)
    return g.reshape(x.shape)


def test_quantize_bytes_bit_exact(nb):
    say("quantize: special groups + skipped/out-of-range slots")
    x = _special_groups()
    T = x.shape[0]
    pages = 3
    rng = np.random.default_rng(1)
    slots = rng.permutation(pages * 128)[:T].astype(np.int64)
    slots[5] = -1
    slots[6] = pages * 128 + 3          # out of range: skipped
    codes, scales = nb.empty_pool(pages, 4)
    codes.fill_(0xAB)
    scales.fill_(0xCD)
    nb.msa_nvfp4_quantize(torch.from_numpy(x).cuda(), torch.from_numpy(slots).cuda(), codes,
                          scales)
    rc, rs = nvfp4.empty_pool(pages, 4)
    rc[:] = 0xAB
    rs[:] = 0xCD
    ok = (slots >= 0) & (slots < pages * 128)
    nvfp4.write_cache(rc, rs, x[ok], slots[ok])
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(nb.scales_rows(scales).cpu().numpy(), rs)


def test_quantize_empty_is_noop(nb):
    codes, scales = nb.empty_pool(1, 4)
    codes.fill_(7)
    nb.msa_nvfp4_quantize(torch.empty((0, 4, 128), device="cuda"),
                          torch.empty(0, dtype=torch.int64, device="cuda"), codes, scales)
    torch.cuda.synchronize()
    assert int(codes.min()) == 7 == int(codes.max())


# ------------------------------------------------------------------ small ragged cases
TINY = [
    ([1, 130, 2177, 4099], 1),
    ([17 * 128, 18 * 128, 17 * 128 + 1, 16 * 128 + 5, 128, 129], 1),
    ([2, 129, 2400, 3000], 2),
    ([3, 300, 2200], 3),
    ([4, 640, 2560 + 1], 4),
    ([5, 700, 2304], 5),
    ([8, 135, 2300, 5000], 8),
    ([8 * 128 + 3, 19 * 128 + 7, 3001], 8),
]


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "separate"])
@pytest.mark.parametrize("lens,q", TINY)
def test_tiny_parity(nb, lens, q, fused):
    say(f"tiny parity lens={lens} q={q} fused={fused}")
    wl = tiny_config(lens, q, seed=sum(lens) + q)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    ids, sc, o = _to_np(S.run_step(nb, wl, pools, inp, fused=fused))
    _structural(wl, ids)
    fails = S.check_page_bytes(wl, pools, np.unique(wl.block_table[wl.block_table >= 0]))
    for b in range(wl.num_seqs):
        fails += S.check_sequence(wl, b, ids, sc, o)
    assert not fails, "\n".join(fails[:20])


# The attention launch plan switches on pairs * slots (pairs = query tokens
# x KV heads, 17 slots): up to 384 workgroups the four wavefronts of a
# workgroup share each block (32 tokens each), above that every wavefront
# takes whole blocks. Five sequences (20 pairs) run the shared form, six
# (24 pairs) the whole-block form, on the same lengths.
@pytest.mark.parametrize("nseq", [5, 6], ids=["shared-block-waves", "whole-block-waves"])
def test_attention_launch_forms(nb, nseq):
    lens = [1, 130, 200, 2177, 4099, 3000][:nseq]
    say(f"attention launch forms lens={lens}")
    wl = tiny_config(lens, 1, seed=60 + nseq)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    for fused in (True, False):
        ids, sc, o = _to_np(S.run_step(nb, wl, pools, inp, fused=fused))
        _structural(wl, ids)
        fails = []
        for b in range(wl.num_seqs):
            fails += S.check_sequence(wl, b, ids, sc, o)
        assert not fails, "\n".join(fails[:20])


# With whole blocks per wavefront the plan takes the number of slots per
# wavefront with the shortest chain among the grids that fit the 512
# workgroups the chip holds at once, else one split per (query token, KV
# head) pair, written directly: 160 pairs run 2 slots per wavefront (3
# splits), 192 pairs and 8 x 8 query tokens (256 pairs) one split.
@pytest.mark.parametrize("nseq,q", [(40, 1), (48, 1), (8, 8)],
                         ids=["2-slots-3-splits", "one-split", "one-split-q8"])
def test_attention_plan_many_pairs(nb, nseq, q):
    rng = np.random.default_rng(nseq * 10 + q)
    lens = [int(x) for x in rng.integers(17 * 128 + 1, 24 * 128, size=nseq)]
    lens[0] = 16 * 128 + 3                        # fewer than 17 blocks: every block
    say(f"attention plan, {nseq} sequences x {q} query tokens")
    wl = tiny_config(lens, q, seed=70 + nseq)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    for fused in (True, False):
        ids, sc, o = _to_np(S.run_step(nb, wl, pools, inp, fused=fused))
        _structural(wl, ids)
        assert np.all(np.isfinite(o))
        fails = []
        for b in (0, 1, nseq // 2, nseq - 1):
            fails += S.check_sequence(wl, b, ids, sc, o)
        assert not fails, "\n".join(fails[:20])


@pytest.mark.parametrize("heads", [1, 2, 8])
def test_head_counts(nb, heads):
    # every kernel takes the number of index-key / KV heads at run time (1..8,
    # 8 query heads each); the scan uses one wavefront per head
    say(f"{heads} index / KV heads, {8 * heads} query heads")
    wl = tiny_config([2400, 700, 17 * 128 + 1], 2, seed=50 + heads)
    wl.num_kv_heads = wl.num_idx_heads = heads
    wl.num_q_heads = 8 * heads
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    ids, sc, o = _to_np(S.run_step(nb, wl, pools, inp))
    ids2, sc2, o2 = _to_np(S.run_step(nb, wl, pools, inp, fused=False))
    assert np.array_equal(ids, ids2) and np.array_equal(o, o2)
    _structural(wl, ids)
    fails = S.check_page_bytes(wl, pools, wl.pages_in_use()[:6])
    for b in range(wl.num_seqs):
        fails += S.check_sequence(wl, b, ids, sc, o)
    assert not fails, "\n".join(fails[:20])


def test_outlier_channels_parity(nb):
    say("tiny parity with 5% outlier channels")
    wl = tiny_config([3000, 4100], 1, seed=5, outliers=True)
    pools = S.fill_pools(wl, nb)
    ids, sc, o = _to_np(S.run_step(nb, wl, pools, S.device_inputs(wl)))
    fails = S.check_page_bytes(wl, pools, wl.pages_in_use())
    for b in range(wl.num_seqs):
        fails += S.check_sequence(wl, b, ids, sc, o)
    assert not fails, "\n".join(fails[:20])


# ------------------------------------------------------------------ planted / ties
def _plant(wl, rows_by_page, coef_by_page):
    """Override: token row r of page p's index key = coef * sum of the query
    heads of each index head's group (strongly aligned with every head)."""
    qv = S.fp8_values(wl.q_idx())[0]          # [32, 128]
    keys = np.stack([qv[8 * g:8 * g + 8].sum(axis=0) for g in range(4)]).astype(np.float32)

    def ov(stream, pages, src):
        if stream != synth.STREAM_IDX:
            return src
        src = src.clone()
        for k, p in enumerate(np.asarray(pages).tolist()):
            if p in rows_by_page:
                r = rows_by_page[p]
                src[k * 128 + r] = torch.from_numpy(keys * coef_by_page[p]).to(src.device)
        return src
    return ov


def test_planted_blocks_and_duplicate_page_tie(nb):
    say("planted blocks + duplicated page tie")
    wl = tiny_config([40 * 128], 1, seed=21, spare_pages=0, permute=False)
    bt = wl.block_table
    # logical blocks 10 and 25 share one physical page (a shared prefix-like alias)
    bt[0, 25] = bt[0, 10]
    planted = [2, 4, 5, 7, 9, 13, 15, 17, 19, 22, 27, 30, 33, 35, 38]   # 15 blocks
    rows = {int(bt[0, j]): (7 * j) % 128 for j in planted + [10]}
    coef = {int(bt[0, j]): 1.0 for j in planted}
    coef[int(bt[0, 10])] = 0.5                      # 16th place, tied between 10 and 25
    ov = _plant(wl, rows, coef)
    pools = S.fill_pools(wl, nb, overrides=ov)
    ids, sc, o = _to_np(S.run_step(nb, wl, pools, S.device_inputs(wl)))
    assert ids[0].tolist() == sorted(planted + [10]) + [39]
    fails = S.check_sequence(wl, 0, ids, sc, o, overrides=ov)
    assert not fails, "\n".join(fails)


# ------------------------------------------------------------------ device-side checks
def test_invalid_lengths_and_pages_do_not_fault(nb):
    say("invalid lengths / page ids")
    wl = tiny_config([3000, 2500, 2600, 2700], 2, seed=8)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    lens = inp["seq_lens"].clone()
    lens[1] = 1                                   # shorter than q_per_seq
    lens[2] = wl.max_blocks * 128 + 1             # longer than the block table
    inp["seq_lens"] = lens
    bt = inp["block_table"].clone()
    bt[3, 2] = wl.num_pages + 7                   # page ids out of range
    bt[3, 5] = -3
    inp["block_table"] = bt
    ids, sc, o = _to_np(S.run_step(nb, wl, pools, inp))
    for b in (1, 2):
        assert np.all(ids[2 * b:2 * b + 2] == -1)
        assert np.all(o[2 * b:2 * b + 2] == 0)
    assert np.all(np.isfinite(o))
    assert np.all(sc[6:8][ids[6:8] == 2] == 0) and np.all(sc[6:8][ids[6:8] == 5] == 0)
    fails = S.check_sequence(wl, 0, ids, sc, o)
    assert not fails, "\n".join(fails)


def test_deterministic_and_reusable_workspace(nb):
    say("determinism over repeated calls with one workspace")
    wl = tiny_config([5000, 3001, 129], 8, seed=3)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    ws_i = nb.indexer_workspace(wl.num_seqs, wl.q_per_seq, wl.max_blocks)
    ws_a = nb.attn_workspace(wl.num_seqs, wl.q_per_seq, wl.num_q_heads, wl.topk + 1)
    first = _to_np(S.run_step(nb, wl, pools, inp, ws_i, ws_a))
    for _ in range(3):
        again = _to_np(S.run_step(nb, wl, pools, inp, ws_i, ws_a))
        for x, y in zip(first, again):
            assert np.array_equal(x, y)


def test_two_stage_indexer_equals_decode(nb):
    say("scan + select == decode")
    wl = tiny_config([5000, 3001, 129, 2200], 3, seed=4)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    ic, isc = pools[synth.STREAM_IDX]
    tq = wl.num_q_tokens
    ws = nb.indexer_workspace(wl.num_seqs, wl.q_per_seq, wl.max_blocks)
    ids1 = torch.empty((tq, 17), dtype=torch.int32, device="cuda")
    sc1 = torch.empty((tq, 17), dtype=torch.float32, device="cuda")
    nb.msa_indexer_decode(ic, isc, inp["q_idx"], inp["w"], inp["block_table"], inp["seq_lens"],
                          wl.q_per_seq, ids1, ws, out_scores=sc1)
    bscores = torch.full((tq, wl.max_blocks), -7.0, dtype=torch.float32, device="cuda")
    nb.msa_indexer_scan(ic, isc, inp["q_idx"], inp["w"], inp["block_table"], inp["seq_lens"],
                        wl.q_per_seq, bscores)
    ids2 = torch.empty_like(ids1)
    sc2 = torch.empty_like(sc1)
    nb.msa_indexer_select(bscores, inp["seq_lens"], wl.q_per_seq, ids2, sc2)
    torch.cuda.synchronize()
    assert torch.equal(ids1, ids2) and torch.equal(sc1, sc2)
    # entries past each query token's visible blocks are left untouched
    bs = bscores.cpu().numpy()
    for b in range(wl.num_seqs):
        for i, pos in enumerate(wl.positions(b)):
            row = b * wl.q_per_seq + i
            nbk = pos // 128 + 1
            assert np.all(bs[row, nbk:] == -7.0) and np.all(bs[row, :nbk] >= 0)


@pytest.mark.parametrize("lens,q", [TINY[1], TINY[3], TINY[7]])
def test_fused_select_attention_equals_separate(nb, lens, q):
    say(f"selection inside attention == select + attention, lens={lens} q={q}")
    wl = tiny_config(lens, q, seed=11 + q, spare_pages=5, permute=True)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    a = _to_np(S.run_step(nb, wl, pools, inp, fused=False))
    b = _to_np(S.run_step(nb, wl, pools, inp, fused=True))
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1], b[1])
    assert np.array_equal(a[2], b[2])          # the same blocks in the same order: same bits


def test_fused_select_attention_without_ids_and_invalid_rows(nb):
    say("selection inside attention: no id output, invalid lengths and pages")
    wl = tiny_config([2500, 3000, 40, 2600], 2, seed=12)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    lens = inp["seq_lens"].clone()
    lens[1] = wl.max_blocks * 128 + 1            # longer than the block table
    lens[2] = 1                                  # shorter than q_per_seq
    bt = inp["block_table"].clone()
    bt[3, 3] = -5
    bt[3, 7] = 1 << 30
    inp = dict(inp, seq_lens=lens, block_table=bt)
    kc, ks = pools[synth.STREAM_K]
    vc, vs = pools[synth.STREAM_V]
    ic, isc = pools[synth.STREAM_IDX]
    tq = wl.num_q_tokens
    bscores = torch.zeros((tq, wl.max_blocks), dtype=torch.float32, device="cuda")
    nb.msa_indexer_scan(ic, isc, inp["q_idx"], inp["w"], bt, lens, wl.q_per_seq, bscores)
    ws = nb.attn_workspace(wl.num_seqs, wl.q_per_seq, wl.num_q_heads, 17)
    o1 = torch.full((tq, 32, 128), 5.0, device="cuda")
    o2 = torch.full((tq, 32, 128), 5.0, device="cuda")
    ids = torch.full((tq, 17), 99, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(128)
    nb.msa_sparse_attn_select_decode(kc, ks, vc, vs, inp["q_attn"], bt, lens, wl.q_per_seq,
                                     bscores, scale, o1, ws)
    nb.msa_sparse_attn_select_decode(kc, ks, vc, vs, inp["q_attn"], bt, lens, wl.q_per_seq,
                                     bscores, scale, o2, ws, out_ids=ids)
    ids_ref = torch.empty_like(ids)
    nb.msa_indexer_select(bscores, lens, wl.q_per_seq, ids_ref)
    o3 = torch.empty_like(o1)
    nb.msa_sparse_attn_decode(kc, ks, vc, vs, inp["q_attn"], bt, lens, wl.q_per_seq, ids_ref,
                              scale, o3, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
    assert torch.equal(ids, ids_ref)
    idn = ids.cpu().numpy()
    on = o1.cpu().numpy()
    for b in (1, 2):
        assert np.all(idn[2 * b:2 * b + 2] == -1)
        assert np.all(on[2 * b:2 * b + 2] == 0)
    assert np.all(np.isfinite(on))


def test_prepared_calls_match_direct(nb):
    say("prepared calls (arguments marshalled once) re-issue the same launches")
    wl = tiny_config([2600, 900], 1, seed=41)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    ref = _to_np(S.run_step(nb, wl, pools, inp))
    ic, isc = pools[synth.STREAM_IDX]
    kc, ks = pools[synth.STREAM_K]
    vc, vs = pools[synth.STREAM_V]
    tq = wl.num_q_tokens
    bscores = torch.empty((tq, wl.max_blocks), dtype=torch.float32, device="cuda")
    ws = nb.attn_workspace(wl.num_seqs, wl.q_per_seq, wl.num_q_heads, 17)
    o = torch.empty((tq, wl.num_q_heads, 128), dtype=torch.float32, device="cuda")
    ids = torch.empty((tq, 17), dtype=torch.int32, device="cuda")
    scan = nb.msa_indexer_scan(ic, isc, inp["q_idx"], inp["w"], inp["block_table"],
                               inp["seq_lens"], wl.q_per_seq, bscores, prepare=True)
    attend = nb.msa_sparse_attn_select_decode(kc, ks, vc, vs, inp["q_attn"], inp["block_table"],
                                              inp["seq_lens"], wl.q_per_seq, bscores,
                                              1.0 / math.sqrt(128), o, ws, out_ids=ids,
                                              prepare=True)
    for rep in range(3):
        o.fill_(float(rep))
        ids.fill_(-5)
        scan()
        attend()
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), ref[0]), rep
        assert np.array_equal(o.cpu().numpy(), ref[2]), rep


def test_graph_replay_matches_eager(nb):
    say("decode step captured in a HIP graph, replayed between eager work")
    wl = tiny_config([3000, 2400, 700], 2, seed=31)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    ws_i = nb.indexer_workspace(wl.num_seqs, wl.q_per_seq, wl.max_blocks)
    ws_a = nb.attn_workspace(wl.num_seqs, wl.q_per_seq, wl.num_q_heads, wl.topk + 1)
    tq = wl.num_q_tokens
    out = dict(ids=torch.empty((tq, 17), dtype=torch.int32, device="cuda"),
               scores=torch.empty((tq, 17), dtype=torch.float32, device="cuda"),
               o=torch.empty((tq, wl.num_q_heads, 128), dtype=torch.float32, device="cuda"))
    ref = _to_np(S.run_step(nb, wl, pools, inp, ws_i, ws_a, out))
    ic, isc = pools[synth.STREAM_IDX]
    kc, ks = pools[synth.STREAM_K]
    vc, vs = pools[synth.STREAM_V]
    bscores = ws_i[: tq * wl.max_blocks * 4].view(torch.float32).view(tq, wl.max_blocks)

    def step():
        nb.msa_indexer_scan(ic, isc, inp["q_idx"], inp["w"], inp["block_table"], inp["seq_lens"],
                            wl.q_per_seq, bscores)
        nb.msa_sparse_attn_select_decode(kc, ks, vc, vs, inp["q_attn"], inp["block_table"],
                                         inp["seq_lens"], wl.q_per_seq, bscores,
                                         1.0 / math.sqrt(128), out["o"], ws_a, out_ids=out["ids"])
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
        cap.synchronize()
        with torch.cuda.graph(g, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    other = tiny_config([1500, 900, 300], 2, seed=32)       # same shapes, other data
    other_inp = S.device_inputs(other)
    for rep in range(3):
        out["o"].fill_(float(rep + 1))
        out["ids"].fill_(-7)
        bscores.fill_(3.0)
        # eager work on other inputs between replays, sharing the workspaces
        S.run_step(nb, other, pools, other_inp, ws_i, ws_a, dict(
            ids=torch.empty_like(out["ids"]), scores=torch.empty_like(out["scores"]),
            o=torch.empty_like(out["o"])))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out["ids"].cpu().numpy(), ref[0]), rep
        assert np.array_equal(out["o"].cpu().numpy(), ref[2]), rep


@pytest.mark.parametrize("mb", [3000, 2050, 2049, 1500, 66, 65, 40, 19, 18])
def test_select_many_equal_scores(nb, mb):
    # 2049 blocks = 2048 candidates, the most held in registers; 2050 and up
    # re-read the scores from memory; 65 blocks (64 candidates) and fewer are
    # ranked directly, 66 and more go through the threshold first
    say(f"selection with random, all-equal and adversarial scores, {mb} blocks")
    tq = 6
    lens = torch.tensor([mb * 128] * tq, dtype=torch.int32, device="cuda")
    bs = _adversarial_scores(mb, tq)
    ids = torch.empty((tq, 17), dtype=torch.int32, device="cuda")
    sc = torch.empty((tq, 17), dtype=torch.float32, device="cuda")
    nb.msa_indexer_select(torch.from_numpy(bs).cuda(), lens, 1, ids, sc)
    torch.cuda.synchronize()
    from oracle import msa
    for r in range(tq):
        want = msa.select_blocks(np.maximum(bs[r].astype(np.float64), 0.0))
        assert ids[r].cpu().numpy().tolist() == want.tolist(), r
        got_sc = sc[r].cpu().numpy()
        want_sc = np.where(want >= 0, np.maximum(bs[r], 0)[np.maximum(want, 0)], 0)
        assert np.array_equal(got_sc, want_sc.astype(np.float32)), r


def _adversarial_scores(mb, tq=6):
    rng = np.random.default_rng(2 + mb)
    bs = np.zeros((tq, mb), dtype=np.float32)
    bs[0] = rng.random(mb, dtype=np.float32)
    bs[1] = np.tile(np.arange(64, dtype=np.float32)[::-1], mb // 64 + 1)[:mb]   # periodic
    bs[2] = rng.integers(0, 3, mb).astype(np.float32)                            # few levels
    bs[3] = -0.0
    bs[4] = np.arange(mb, dtype=np.float32)                                      # ascending
    bs[5] = rng.random(mb, dtype=np.float32)
    bs[5, rng.choice(mb - 1, min(40, mb - 1), replace=False)] = 2.0             # 40-way tie on top
    return bs


@pytest.mark.parametrize("rows", [(0, 1, 2, 3, 4, 5), (1, 3, 5)], ids=["whole-block", "shared-block"])
@pytest.mark.parametrize("mb", [3000, 2050, 2049, 1500, 66, 65])
def test_fused_select_many_equal_scores(nb, mb, rows):
    # The selection inside the attention launch on adversarial score rows.
    # 66..2049 blocks: the workgroup's shared selection, and with the
    # periodic and all-zero rows (hundreds of candidates reach the
    # threshold) its fall-back to one wavefront's exact rounds; 2050 and up:
    # the per-wavefront selection over several chunks; 65: direct ranking.
    # Six query tokens (24 pairs x 17 slots) take the whole-block launch
    # form, three (12 pairs) the shared-block form.
    say(f"selection inside attention, adversarial scores, {mb} blocks, rows {rows}")
    tq, pages = len(rows), 8
    bs = np.ascontiguousarray(_adversarial_scores(mb)[list(rows)])
    lens = torch.tensor([mb * 128] * tq, dtype=torch.int32, device="cuda")
    table = (torch.arange(mb, dtype=torch.int32) % pages).repeat(tq, 1).contiguous().cuda()
    codes = torch.zeros((pages, 4, 128, 64), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((pages, 4, 1024), dtype=torch.uint8, device="cuda")
    q = torch.zeros((tq, 32, 128), dtype=torch.uint8, device="cuda")
    out = torch.full((tq, 32, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = nb.attn_workspace(tq, 1, 32, 17)
    ids = torch.empty((tq, 17), dtype=torch.int32, device="cuda")
    bst = torch.from_numpy(bs).cuda()
    nb.msa_sparse_attn_select_decode(codes, scales, codes, scales, q, table, lens, 1, bst,
                                     1.0 / math.sqrt(128.0), out, ws, out_ids=ids)
    ids2 = torch.empty((tq, 17), dtype=torch.int32, device="cuda")
    sc = torch.empty((tq, 17), dtype=torch.float32, device="cuda")
    nb.msa_indexer_select(bst, lens, 1, ids2, sc)
    torch.cuda.synchronize()
    from oracle import msa
    for r in range(tq):
        want = msa.select_blocks(np.maximum(bs[r].astype(np.float64), 0.0))
        assert ids[r].cpu().numpy().tolist() == want.tolist(), r
    assert torch.equal(ids, ids2)
    # zero K and V: every selected block contributes zero
    assert torch.equal(out, torch.zeros_like(out))


def test_empty_batch_and_bad_shapes(nb):
    wl = tiny_config([300], 1)
    pools = S.fill_pools(wl, nb)
    ic, isc = pools[synth.STREAM_IDX]
    z = torch.empty((0, 32, 128), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    nb.msa_indexer_decode(ic, isc, z, torch.empty((0, 32), device="cuda"),
                          torch.empty((0, 4), dtype=torch.int32, device="cuda"),
                          torch.empty(0, dtype=torch.int32, device="cuda"), 1,
                          torch.empty((0, 17), dtype=torch.int32, device="cuda"), ws)
    inp = S.device_inputs(wl)
    with pytest.raises(nb.MsaError):
        nb.msa_indexer_decode(ic, isc, inp["q_idx"], inp["w"], inp["block_table"],
                              inp["seq_lens"], 1,
                              torch.empty((1, 17), dtype=torch.int32, device="cuda"),
                              torch.zeros(16, dtype=torch.uint8, device="cuda"))


# ------------------------------------------------------------------ the five workloads
# Sequences checked against the oracle in full (block scores, selection,
# attention); every query token's ids are checked for structure, and the
# selection inside the attention launch against the standalone selection.
# The fp64 oracle takes ~6 s per 2,048 blocks of one query token.
SAMPLES = {0: [0], 1: [0, 7, 19, 31], 2: [0, 3, 5, 7], 3: [2, 11, 15], 4: None}


@pytest.mark.parametrize("ci", [0, 1, 2, 3, 4])
def test_workload_parity(nb, ci):
    wl = get_config(ci)
    say(f"workload {ci} {wl.name}: filling pools")
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    say(f"workload {ci}: decode step")
    ids, sc, o = _to_np(S.run_step(nb, wl, pools, inp))
    _structural(wl, ids)
    assert np.all(np.isfinite(o))
    seqs = SAMPLES[ci]
    if seqs is None:                               # shortest and longest request
        seqs = [int(np.argmin(wl.seq_lens)), int(np.argmax(wl.seq_lens))]
    rng = np.random.default_rng(ci)
    used = wl.pages_in_use()
    pages = rng.choice(used, size=min(6, len(used)), replace=False)
    say(f"workload {ci}: page bytes {pages.tolist()}")
    fails = S.check_page_bytes(wl, pools, pages)
    for b in seqs:
        say(f"workload {ci}: oracle on sequence {b} (length {wl.seq_lens[b]})")
        fails += S.check_sequence(wl, b, ids, sc, o)
    assert not fails, "\n".join(fails[:20])


# Shared-prefix scan: groups of sequences whose leading blocks map to the
# same pages (derived by the library from the block table) are scored with
# one read and one dequantisation per shared block, in the scan's own
# launch; the block scores must be the plain scan's, bit for bit, and the
# decode on them must pass the oracle. Cases: a member whose last shared
# block is only partly visible (L = 130, Q = 2), two groups plus an
# ungrouped sequence, nine members with Q = 1, three members with Q = 8,
# and 70 members (two chunks of 64 sequences in a shared workgroup).
SHARED = [
    ([1000, 700, 3000, 130, 2600, 900], 2, [([0, 1, 3], 6), ([2, 4], 20)]),
    ([2300] * 9 + [500], 1, [(list(range(9)), 17)]),
    ([4100, 4000, 3000], 8, [([0, 1, 2], 23)]),
    ([700 + 13 * i for i in range(70)], 1, [(list(range(70)), 5)]),
]


def _plain_and_shared(nb, wl, inp, pools, groups):
    ic, isc = pools[synth.STREAM_IDX]
    tq = wl.num_q_tokens
    ref = torch.full((tq, wl.max_blocks), -1.0, dtype=torch.float32, device="cuda")
    got = torch.full((tq, wl.max_blocks), -2.0, dtype=torch.float32, device="cuda")
    nb.msa_indexer_scan(ic, isc, inp["q_idx"], inp["w"], inp["block_table"], inp["seq_lens"],
                        wl.q_per_seq, ref)
    nb.msa_indexer_scan_shared(ic, isc, inp["q_idx"], inp["w"], inp["block_table"],
                               inp["seq_lens"], wl.q_per_seq, *groups, got)
    torch.cuda.synchronize()
    ref_np, got_np = ref.cpu().numpy(), got.cpu().numpy()
    lens = inp["seq_lens"].cpu().numpy()          # the lengths the kernels saw
    Q = wl.q_per_seq
    for b in range(wl.num_seqs):
        L = int(lens[b])
        if not Q <= L <= wl.max_blocks * 128:      # invalid length: neither writes the rows
            assert np.all(ref_np[b * Q:(b + 1) * Q] == -1.0)
            assert np.all(got_np[b * Q:(b + 1) * Q] == -2.0), f"seq {b}: written despite its length"
            continue
        for i in range(Q):
            r = b * Q + i
            nbk = (L - Q + i) // 128 + 1
            assert np.array_equal(ref_np[r, :nbk].view(np.uint32), got_np[r, :nbk].view(np.uint32)), \
                f"seq {b} token {i}: shared-prefix scores differ from the plain scan"
    return got


@pytest.mark.parametrize("lens,q,shared", SHARED, ids=["two-groups", "nine", "q8", "seventy"])
def test_shared_prefix_scan(nb, lens, q, shared):
    from msa_workloads.device import shared_groups
    say(f"shared prefix scan {len(lens)} sequences q={q} shared={[(len(m), n) for m, n in shared]}")
    wl = tiny_config(lens, q, seed=70 + q, shared=shared)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    groups = shared_groups(wl, nb)
    assert groups[2] > 0 and len(groups[0]) == len(shared)
    got = _plain_and_shared(nb, wl, inp, pools, groups)
    # the decode step on the shared-prefix scores, against the oracle
    tq = wl.num_q_tokens
    ids = torch.empty((tq, wl.topk + 1), dtype=torch.int32, device="cuda")
    sc = torch.empty((tq, wl.topk + 1), dtype=torch.float32, device="cuda")
    o = torch.empty((tq, wl.num_q_heads, 128), dtype=torch.float32, device="cuda")
    kc, ks = pools[synth.STREAM_K]
    vc, vs = pools[synth.STREAM_V]
    ws = nb.attn_workspace(wl.num_seqs, q, wl.num_q_heads, wl.topk + 1)
    nb.msa_sparse_attn_select_decode(kc, ks, vc, vs, inp["q_attn"], inp["block_table"],
                                     inp["seq_lens"], q, got, 1.0 / math.sqrt(128), o, ws,
                                     out_ids=ids)
    nb.msa_indexer_select(got, inp["seq_lens"], q, torch.empty_like(ids), sc)
    ids_np, sc_np, o_np = _to_np(dict(ids=ids, scores=sc, o=o))
    _structural(wl, ids_np)
    fails = []
    for b in sorted({0, 1, wl.num_seqs // 2, wl.num_seqs - 1}):
        fails += S.check_sequence(wl, b, ids_np, sc_np, o_np)
    assert not fails, "\n".join(fails[:20])


def test_shared_prefix_scan_with_wrong_groups(nb):
    """Group arrays that do not match the block table only share less: a
    member whose pages differ from the lead's, a lead outside the batch, a
    group id past num_groups, a group longer than the table, a sequence of
    invalid length in a group, and a member listed in a group it does not
    share pages with. Every score must still be the plain scan's."""
    say("shared prefix scan with group arrays that do not match the block table")
    wl = tiny_config([3000, 2600, 2900, 2500, 1900, 3100], 2, seed=81,
                     shared=[([0, 1, 2], 12), ([3, 4], 9)])
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    lens = inp["seq_lens"].clone()
    lens[4] = 1                                   # invalid length, still in group 1
    inp["seq_lens"] = lens
    i32 = dict(dtype=torch.int32, device="cuda")
    lead = torch.tensor([0, 3, 77], **i32)         # group 2: lead outside the batch
    blocks = torch.tensor([14, 40, 5], **i32)      # group 0 claims 14 (12 shared), group 1 past the table
    seq_group = torch.tensor([0, 0, 0, 1, 1, 0], **i32)   # seq 5 shares nothing with the lead
    _plain_and_shared(nb, wl, inp, pools, (lead, blocks, wl.max_blocks, seq_group))
    seq_group = torch.tensor([2, 5, 0, -1, 1, 1], **i32)  # ids past num_groups, the lead outside
    _plain_and_shared(nb, wl, inp, pools, (lead, blocks, wl.max_blocks, seq_group))


def test_shared_prefix_scan_without_groups_is_plain_scan(nb):
    say("shared prefix scan, no groups")
    wl = tiny_config([2000, 900, 130], 2, seed=77)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    ic, isc = pools[synth.STREAM_IDX]
    tq = wl.num_q_tokens
    ref = torch.full((tq, wl.max_blocks), -1.0, dtype=torch.float32, device="cuda")
    got = torch.full((tq, wl.max_blocks), -1.0, dtype=torch.float32, device="cuda")
    nb.msa_indexer_scan(ic, isc, inp["q_idx"], inp["w"], inp["block_table"], inp["seq_lens"], 2, ref)
    i32 = dict(dtype=torch.int32, device="cuda")
    nb.msa_indexer_scan_shared(ic, isc, inp["q_idx"], inp["w"], inp["block_table"],
                               inp["seq_lens"], 2, torch.zeros(0, **i32), torch.zeros(0, **i32), 0,
                               torch.full((wl.num_seqs,), -1, **i32), got)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int32), got.view(torch.int32))


@pytest.mark.parametrize("q", [1, 2])
def test_scan_scores_independent_of_grid(nb, q):
    """The block scores of a batch large enough for the scan grid's trailing
    one-block workgroups (44 sequences of up to 256 blocks: 44 x 86 regular
    workgroups, more than two rounds of the chip) equal, bit for bit, those
    of scanning each sequence alone (a one-sequence grid of 86 workgroups,
    no trailing rows): every block is scored once, by the same arithmetic,
    whichever workgroup takes it."""
    lens = [32768 - 97 * b for b in range(44)]
    say(f"scan scores independent of the grid, 44 sequences up to 32K, q={q}")
    wl = tiny_config(lens, q, seed=90 + q, spare_pages=3, permute=True)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    ic, isc = pools[synth.STREAM_IDX]
    tq = wl.num_q_tokens
    whole = torch.full((tq, wl.max_blocks), -3.0, dtype=torch.float32, device="cuda")
    nb.msa_indexer_scan(ic, isc, inp["q_idx"], inp["w"], inp["block_table"], inp["seq_lens"], q,
                        whole)
    alone = torch.full_like(whole, -3.0)
    hq = wl.num_q_heads
    for b in range(wl.num_seqs):
        rows = slice(b * q, (b + 1) * q)
        nb.msa_indexer_scan(ic, isc, inp["q_idx"][rows].contiguous(), inp["w"][rows].contiguous(),
                            inp["block_table"][b:b + 1].contiguous(),
                            inp["seq_lens"][b:b + 1].contiguous(), q, alone[rows])
    torch.cuda.synchronize()
    assert inp["q_idx"].shape[1] == hq
    assert torch.equal(whole.view(torch.int32), alone.view(torch.int32))
    # every visible block has a score; nothing past the visible blocks is written
    bs = whole.cpu().numpy()
    for b in range(wl.num_seqs):
        for i, pos in enumerate(wl.positions(b)):
            nbk = pos // 128 + 1
            assert np.all(bs[b * q + i, :nbk] >= 0) and np.all(bs[b * q + i, nbk:] == -3.0)


# msa_sparse_attn_decode with the caller's selection and num_sel from 1 to
# 64 slots, through each form of the launch plan: one workgroup per slot
# (the four wavefronts share each block) while pairs x num_sel <= 384, else
# whole blocks per wavefront with R slots per wavefront and the split merge,
# or one split per pair written directly. (num_sel, lengths, query tokens
# per sequence, plan exercised.)
def _numsel_lens(n, lo, hi, seed):
    return [int(x) for x in np.random.default_rng(seed).integers(lo, hi, size=n)]


NUMSEL = [
    (1, [3000, 700, 129], 1, "shared-block waves"),
    (1, _numsel_lens(100, 300, 700, 1), 1, "whole blocks, 1 slot per wave"),
    (5, [3000, 2000, 129, 40], 2, "shared-block waves"),
    (5, _numsel_lens(25, 1000, 3000, 2), 1, "whole blocks, 2 splits"),
    (33, [5000, 4000], 1, "shared-block waves, 33 partials merged"),
    (33, [5000, 4000, 3000], 1, "whole blocks, 9 splits"),
    (33, _numsel_lens(16, 4300, 6000, 3), 1, "whole blocks, 3 slots per wave, 3 splits"),
    (33, [5000, 4300], 4, "whole blocks, 9 splits, 4 query tokens"),
    (64, [9000], 1, "shared-block waves, 64 partials merged"),
    (64, [9000, 8500], 1, "whole blocks, 16 splits"),
    (64, _numsel_lens(12, 8300, 9500, 4), 1, "whole blocks, 2 slots per wave, 8 splits"),
    (64, _numsel_lens(40, 8300, 9000, 5), 1, "whole blocks, 6 slots per wave, 3 splits"),
    (64, _numsel_lens(96, 8300, 9000, 6), 1, "whole blocks, one split of 16 slots per wave"),
]


def _numsel_ids(wl, num_sel, rng):
    """int32 [T_q, num_sel]: distinct visible blocks in random order; some
    rows also hold entries the kernel must ignore (-1, a block past the
    query token's position, a block past the block table), and one row
    holds nothing usable."""
    ids = np.full((wl.num_q_tokens, num_sel), -1, dtype=np.int32)
    for b in range(wl.num_seqs):
        for i, pos in enumerate(wl.positions(b)):
            r = b * wl.q_per_seq + i
            nvis = pos // 128 + 1
            junk = []
            if num_sel >= 4 and r % 3 == 1:
                junk = [-1, wl.max_blocks + 3]
                if nvis < wl.max_blocks:
                    junk.append(nvis)              # past this token's position
            k = min(num_sel - len(junk), nvis)
            row = list(rng.choice(nvis, size=k, replace=False)) + junk
            rng.shuffle(row)
            ids[r, :len(row)] = row
    if wl.num_q_tokens > 2:
        ids[2] = -1                                # nothing usable: zero output
        ids[2, 0] = wl.max_blocks + 1
    return ids


@pytest.mark.parametrize("num_sel,lens,q,plan", NUMSEL,
                         ids=[f"{n}sel-{len(ls)}x{q}-{p.split(',')[0].replace(' ', '_')}"
                              for n, ls, q, p in NUMSEL])
def test_attention_num_sel(nb, num_sel, lens, q, plan):
    from oracle import msa
    from oracle.acceptance import attention_error, check_attention
    say(f"msa_sparse_attn_decode num_sel={num_sel}, {len(lens)} sequences x {q}: {plan}")
    wl = tiny_config(lens, q, seed=300 + num_sel + len(lens))
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    rng = np.random.default_rng(num_sel * 1000 + len(lens))
    ids = _numsel_ids(wl, num_sel, rng)
    kc, ks = pools[synth.STREAM_K]
    vc, vs = pools[synth.STREAM_V]
    tq = wl.num_q_tokens
    ws = nb.attn_workspace(wl.num_seqs, q, wl.num_q_heads, num_sel)
    o = torch.full((tq, wl.num_q_heads, 128), float("nan"), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(128)
    nb.msa_sparse_attn_decode(kc, ks, vc, vs, inp["q_attn"], inp["block_table"], inp["seq_lens"],
                              q, torch.from_numpy(ids).cuda(), scale, o, ws)
    torch.cuda.synchronize()
    on = o.cpu().numpy()
    assert np.all(np.isfinite(on))
    if tq > 2:
        assert np.all(on[2] == 0)
    q_attn = S.fp8_values(wl.q_attn())
    seqs = sorted({0, 1 % wl.num_seqs, wl.num_seqs // 2, wl.num_seqs - 1})
    fails, errs = [], []
    for b in seqs:
        rows = [b * q + i for i in range(q)]
        blocks = [int(x) for r in rows for x in ids[r] if 0 <= x < wl.blocks_of(b)]
        kv = S.oracle_kv(wl, b, blocks)
        for i, pos in enumerate(wl.positions(b)):
            r = rows[i]
            if r == 2 and tq > 2:
                continue
            ref = msa.sparse_attention(q_attn[r], kv[synth.STREAM_K], kv[synth.STREAM_V], ids[r],
                                       pos, scale)
            errs.append(attention_error(on[r], ref))
            msg = check_attention(on[r], ref)
            if msg:
                fails.append(f"seq {b} q {i}: {msg}")
    S.record_attention_error(f"num_sel {num_sel}, {plan}", errs)
    assert not fails, "\n".join(fails[:20])
