"""The one-launch decode step (msa_decode_mono) through the C ABI.

Its block scores, ids and output must equal, bit for bit, those of the
launch sequence bench.py times (msa_indexer_scan + msa_sparse_attn_select_decode)
whenever that sequence runs one workgroup per selected block (query tokens x
4 KV heads x 17 <= 384), and pass the oracle's acceptance rules on every case;
repeated calls on one workspace must give the same bits and leave the
launch's counters at zero.
"""
import math

import numpy as np
import pytest
import torch

import _support as S
from msa_workloads import get_config, synth, tiny_config

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def nb():
    import nvfp4_kv_cache_amd as m
    m.lib()
    return m


def _run_mono(nb, wl, pools, inp, ws=None):
    tq = wl.num_q_tokens
    dev = inp["q_idx"].device
    if ws is None:
        ws = nb.mono_workspace(wl.num_seqs, wl.q_per_seq, wl.num_q_heads, wl.max_blocks, device=dev)
    ids = torch.full((tq, wl.topk + 1), -7, dtype=torch.int32, device=dev)
    o = torch.full((tq, wl.num_q_heads, 128), float("nan"), dtype=torch.float32, device=dev)
    ic, isc = pools[synth.STREAM_IDX]
    kc, ks = pools[synth.STREAM_K]
    vc, vs = pools[synth.STREAM_V]
    nb.msa_decode_mono(ic, isc, inp["q_idx"], inp["w"], kc, ks, vc, vs, inp["q_attn"],
                       inp["block_table"], inp["seq_lens"], wl.q_per_seq, 1.0 / math.sqrt(128), o,
                       ws, out_ids=ids)
    torch.cuda.synchronize()
    bsc = nb.mono_block_scores(ws, wl.num_seqs, wl.q_per_seq, wl.max_blocks)
    return ids.cpu().numpy(), bsc.cpu().numpy().copy(), o.cpu().numpy(), ws


def _sync_region_zero(ws, wl):
    """The launch's counters (last bytes of the workspace) are all zero."""
    # per sequence and per (query token, KV head) pair: 8 counters 16 words
    # apart; per sequence: one more counter; then the error word
    words = (wl.num_seqs + wl.num_q_tokens * 4) * 128 + wl.num_seqs * 16 + 1
    region = -(-words * 4 // 256) * 256
    tail = ws[-region:].cpu().numpy()
    return not tail.any()


def _visible_scores(wl, bsc):
    """Block scores each query token can see (entries past its last block are
    not written by either path)."""
    out = []
    for b in range(wl.num_seqs):
        for i, pos in enumerate(wl.positions(b)):
            out.append(bsc[b * wl.q_per_seq + i, : pos // 128 + 1])
    return out


def _selected_scores(ids, bsc):
    sc = np.zeros(ids.shape, dtype=np.float32)
    for r in range(ids.shape[0]):
        v = ids[r] >= 0
        sc[r][v] = bsc[r][ids[r][v]]
    return sc


def _check(nb, wl, bitwise):
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    ids, bsc, o, ws = _run_mono(nb, wl, pools, inp)
    assert np.all(np.isfinite(o))
    assert _sync_region_zero(ws, wl), "counters not reset"
    if bitwise:
        ref = S.run_step(nb, wl, pools, inp)
        torch.cuda.synchronize()
        rid, ro = ref["ids"].cpu().numpy(), ref["o"].cpu().numpy()
        tq = wl.num_q_tokens
        assert np.array_equal(ids, rid), "ids differ from the two-launch path"
        assert np.array_equal(o.view(np.uint32), ro.view(np.uint32)), \
            "output bits differ from the two-launch path"
        assert tq * 4 * (wl.topk + 1) <= 384
    fails = []
    sc = _selected_scores(ids, bsc)
    for b in range(wl.num_seqs):
        fails += S.check_sequence(wl, b, ids, sc, o)
    return fails, (ids, bsc, o, ws, pools, inp)


# ragged lengths across block edges; query tokens per sequence 1..8
MONO_CASES = [
    ([4096], 1, True),
    ([1, 130, 2177, 4099], 1, True),
    ([17 * 128, 18 * 128, 17 * 128 + 1, 16 * 128 + 5], 1, True),
    ([2, 2400], 2, True),
    ([300, 2200], 2, True),
    ([5, 2304], 2, True),
    ([3, 4000], 3, False),
    ([3900], 8, False),
    ([8 * 128 + 3, 19 * 128 + 7], 4, False),
    # more than 64 candidates: the selection's threshold and compaction on
    # device-scope score loads, up to the entry point's bound of 1,024 block
    # workgroups (1 x 32K, 2 x 16K with one query token)
    ([16384], 1, True),
    ([32768], 1, True),
    ([16384, 16384 - 37], 1, True),
]


@pytest.mark.parametrize("lens,q,bitwise", MONO_CASES)
def test_mono_parity(nb, lens, q, bitwise):
    say(f"mono parity lens={lens} q={q} bitwise={bitwise}")
    wl = tiny_config(lens, q, seed=7 * sum(lens) + q)
    fails, _ = _check(nb, wl, bitwise)
    assert not fails, "\n".join(fails[:20])


def test_mono_scores_equal_scan(nb):
    say("mono block scores vs msa_indexer_scan")
    wl = tiny_config([3000, 1200, 4100], 1, seed=41)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    _, bsc, _, _ = _run_mono(nb, wl, pools, inp)
    ref = torch.empty((wl.num_q_tokens, wl.max_blocks), dtype=torch.float32, device="cuda")
    ic, isc = pools[synth.STREAM_IDX]
    nb.msa_indexer_scan(ic, isc, inp["q_idx"], inp["w"], inp["block_table"], inp["seq_lens"],
                        wl.q_per_seq, ref)
    torch.cuda.synchronize()
    for a, r in zip(_visible_scores(wl, bsc), _visible_scores(wl, ref.cpu().numpy())):
        assert np.array_equal(a.view(np.uint32), r.view(np.uint32))


def test_mono_repeated_calls_and_counters(nb):
    say("mono repeated calls on one workspace")
    wl = tiny_config([2500, 4000, 700], 1, seed=5)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    first = _run_mono(nb, wl, pools, inp)
    ws = first[3]
    for _ in range(4):
        again = _run_mono(nb, wl, pools, inp, ws)
        for x, y in zip(first[:3], again[:3]):
            assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                  y.view(np.uint32) if y.dtype == np.float32 else y)
        assert _sync_region_zero(ws, wl)
    # a smaller batch on a fresh workspace, then the larger one again
    wl2 = tiny_config([900], 2, seed=6)
    fails, _ = _check(nb, wl2, True)
    assert not fails, "\n".join(fails)
    again = _run_mono(nb, wl, pools, inp, ws)
    assert np.array_equal(first[0], again[0])


def test_mono_invalid_lengths_and_pages(nb):
    say("mono invalid lengths / page ids vs the two-launch path")
    wl = tiny_config([3000, 2500, 2600, 2700], 1, seed=8)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    lens = inp["seq_lens"].clone()
    lens[1] = 0                                   # shorter than q_per_seq
    lens[2] = wl.max_blocks * 128 + 1             # longer than the block table
    inp["seq_lens"] = lens
    bt = inp["block_table"].clone()
    bt[3, 2] = wl.num_pages + 7                   # page ids out of range
    bt[3, 5] = -3
    inp["block_table"] = bt
    ids, bsc, o, ws = _run_mono(nb, wl, pools, inp)
    ref = S.run_step(nb, wl, pools, inp)
    torch.cuda.synchronize()
    assert np.array_equal(ids, ref["ids"].cpu().numpy())
    assert np.array_equal(o.view(np.uint32), ref["o"].cpu().numpy().view(np.uint32))
    for b in (1, 2):
        assert np.all(ids[b] == -1) and np.all(o[b] == 0)
    assert _sync_region_zero(ws, wl)


def test_mono_full_size_tiny_workload(nb):
    """The 1 x 4,096-token workload at its real size, in the launch bench.py
    --mono times: bit-identical to the two-launch step, oracle-checked."""
    wl = get_config(0)
    say(f"mono on {wl.name}")
    fails, _ = _check(nb, wl, True)
    assert not fails, "\n".join(fails)


def test_mono_many_equal_scores(nb):
    """1 x 16K where 120 of the 127 candidate blocks alias one physical page,
    so more than 64 candidates tie at the threshold and the selection ranks
    them by arg-max rounds on device-scope loads: the lowest aliased blocks
    win the ties, bit-identical to the two-launch path."""
    say("mono with 120 tied candidates (aliased page)")
    wl = tiny_config([16384], 1, seed=91, spare_pages=0, permute=False)
    bt = wl.block_table
    bt[0, 7:127] = bt[0, 3]                     # blocks 3 and 7..126 share a page
    fails, (ids, bsc, o, ws, pools, inp) = _check(nb, wl, True)
    assert not fails, "\n".join(fails)
    sc = bsc[0, :127]
    assert np.count_nonzero(sc == sc[3]) == 121
    want = sorted(int(x) for x in np.lexsort((np.arange(127), -sc))[:16]) + [127]
    assert ids[0].tolist() == want


def test_mono_error_word_raises_and_resets_counters(nb):
    """The binding reads the launch's error word after a direct call; a set
    word (a bounded wait that timed out) raises MsaError and zeroes the whole
    counter region, so the next call starts from zero counters. The timeout
    is simulated from the host by setting the word and a stale counter."""
    say("mono error word: raise and reset")
    wl = tiny_config([2500, 700], 1, seed=17)
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    ids, bsc, o, ws = _run_mono(nb, wl, pools, inp)
    n = nb.msa_decode_mono_workspace_bytes(wl.num_seqs, 1, wl.num_q_heads, wl.max_blocks)
    ws[n - 4:n].view(torch.int32).fill_(1)          # error word
    ws[n - 256:n - 252].view(torch.int32).fill_(3)   # a stale arrival in the counter region
    with pytest.raises(nb.MsaError, match="timed out"):
        nb.mono_check(ws, wl.num_seqs, 1, wl.num_q_heads, wl.max_blocks)
    assert _sync_region_zero(ws, wl)
    again = _run_mono(nb, wl, pools, inp, ws)
    assert np.array_equal(again[0], ids)
    assert np.array_equal(again[2].view(np.uint32), o.view(np.uint32))
