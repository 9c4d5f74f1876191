"""msa_indexer_decode_noalloc (block scores in the library's own device
array, no workspace) through the C ABI: bit for bit the ids and scores of
msa_indexer_decode with a caller workspace, on two calls in a row, the
second with a smaller batch (the array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import _support as S
from msa_workloads import synth, tiny_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nb():
    import nvfp4_kv_cache_amd as m
    m.lib()
    return m


def _both(nb, wl):
    pools = S.fill_pools(wl, nb)
    inp = S.device_inputs(wl)
    ic, isc = pools[synth.STREAM_IDX]
    tq = wl.num_q_tokens
    ids1 = torch.full((tq, 17), -5, dtype=torch.int32, device="cuda")
    sc1 = torch.full((tq, 17), -5.0, dtype=torch.float32, device="cuda")
    ids2, sc2 = ids1.clone(), sc1.clone()
    ws = nb.indexer_workspace(wl.num_seqs, wl.q_per_seq, wl.max_blocks)
    nb.msa_indexer_decode(ic, isc, inp["q_idx"], inp["w"], inp["block_table"], inp["seq_lens"],
                          wl.q_per_seq, ids1, ws, out_scores=sc1)
    nb.msa_indexer_decode_noalloc(ic, isc, inp["q_idx"], inp["w"], inp["block_table"],
                                  inp["seq_lens"], wl.q_per_seq, ids2, out_scores=sc2)
    torch.cuda.synchronize()
    return ids1.cpu().numpy(), sc1.cpu().numpy(), ids2.cpu().numpy(), sc2.cpu().numpy()


def test_noalloc_matches_workspace_entry_point(nb):
    # a larger batch first (8 query tokens per sequence, 2,000+ blocks per
    # sequence in one of them), then a smaller one: its scores must not be
    # mixed with the stale rows the first call left in the array
    for lens, q, seed in (([300000, 5000, 3001, 129], 3, 4), ([900, 2400], 1, 5)):
        print(f"noalloc vs workspace: lens={lens} q={q}", flush=True)
        wl = tiny_config(lens, q, seed=seed)
        assert wl.num_q_tokens * wl.max_blocks <= nb.NOALLOC_MAX_SCORES
        ids1, sc1, ids2, sc2 = _both(nb, wl)
        assert np.array_equal(ids1, ids2)
        assert np.array_equal(sc1.view(np.uint32), sc2.view(np.uint32))
        assert np.all(ids1.max(axis=1) >= 0)        # every query token selected blocks


def test_noalloc_rejects_more_scores_than_the_array_holds(nb):
    # 1,024 blocks x 1,025 query tokens > 2^20 scores: rejected on the host,
    # nothing launched
    wl = tiny_config([128], 1, seed=1)
    pools = S.fill_pools(wl, nb)
    ic, isc = pools[synth.STREAM_IDX]
    tq, mb = 1025, 1024
    q = torch.zeros((tq, 32, 128), dtype=torch.uint8, device="cuda")
    w = torch.zeros((tq, 32), dtype=torch.float32, device="cuda")
    bt = torch.zeros((tq, mb), dtype=torch.int32, device="cuda")
    lens = torch.ones(tq, dtype=torch.int32, device="cuda")
    ids = torch.empty((tq, 17), dtype=torch.int32, device="cuda")
    with pytest.raises(nb.MsaError, match="workspace"):
        nb.msa_indexer_decode_noalloc(ic, isc, q, w, bt, lens, 1, ids)
