"""Pins of oracle.msa: selection by brute force and invariants, the pages'
block counts, planted blocks, and attention against a library special case
(torch scaled_dot_product_attention in fp64 when every block is selected)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import msa, nvfp4, formats
from oracle.acceptance import check_selection

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))
TOPK = GOLD["selected_blocks"]["value"]
BLOCK = GOLD["block_tokens"]["value"]


def _brute_select(b, topk=TOPK):
    nb = len(b)
    if nb <= topk + 1:
        return list(range(nb)) + [-1] * (topk + 1 - nb)
    best = sorted(range(nb - 1), key=lambda i: (-b[i], i))[:topk]
    return sorted(best) + [nb - 1]


@pytest.mark.parametrize("nb", [1, 2, 16, 17, 18, 19, 40, 300])
def test_select_blocks_brute_force(nb):
    rng = np.random.default_rng(nb)
    for _ in range(20):
        b = rng.integers(0, 6, nb).astype(np.float64)      # many exact ties
        assert msa.select_blocks(b, TOPK).tolist() == _brute_select(b.tolist())
        b = rng.random(nb)
        assert msa.select_blocks(b, TOPK).tolist() == _brute_select(b.tolist())


def test_selection_counts_from_pages():
    # 16 blocks plus the most recent one: 17 blocks of 128 tokens, "roughly 2,048 keys"
    b = np.random.default_rng(1).random(2048)
    ids = msa.select_blocks(b, TOPK)
    assert len(set(ids.tolist())) == TOPK + GOLD["recent_blocks_kept"]["value"]
    assert ids[-1] == 2047
    keys = len(ids) * BLOCK
    assert abs(keys - GOLD["keys_per_query_approx"]["value"]) / 2048 < 0.07


def test_ties_go_to_lower_block_and_recent_always_kept():
    b = np.ones(100)
    ids = msa.select_blocks(b, TOPK)
    assert ids.tolist() == list(range(16)) + [99]
    b = np.zeros(50)
    b[-1] = -5                          # the recent block is kept whatever its score
    assert msa.select_blocks(b, TOPK)[-1] == 49


def test_dcp_shard_merge_equals_global():
    # context sharded four ways, local top-16 per shard, merged: exact selection
    rng = np.random.default_rng(3)
    for nb in (100, 1025, 2048):
        b = rng.random(nb)
        b[rng.integers(0, nb - 1, 30)] = b[0]           # some ties across shards
        cand = np.arange(nb - 1)
        shards = np.array_split(cand, 4)
        local = []
        for sh in shards:
            order = np.lexsort((sh, -b[sh]))
            local.extend(sh[order[:TOPK]].tolist())
        local = np.array(local)
        order = np.lexsort((local, -b[local]))
        merged = sorted(local[order[:TOPK]].tolist()) + [nb - 1]
        assert merged == msa.select_blocks(b, TOPK).tolist()


def _rand_fp8_values(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return formats.e4m3_decode(formats.e4m3_encode(x.astype(np.float64)))


def test_selection_invariant_to_positive_weight_scale():
    rng = np.random.default_rng(4)
    q = _rand_fp8_values(rng, (32, 128))
    k = _rand_fp8_values(rng, (3000, 4, 128))
    w = rng.random(32)
    pos = 2999
    a, _ = msa.indexer(q, w, k, pos)
    b, _ = msa.indexer(q, w * 7.5, k, pos)
    assert np.array_equal(a, b)


def test_planted_blocks_are_selected():
    rng = np.random.default_rng(5)
    q = _rand_fp8_values(rng, (32, 128))
    k = _rand_fp8_values(rng, (40 * BLOCK, 4, 128)) * 0.1
    w = rng.random(32)
    planted = sorted(rng.choice(39, 16, replace=False).tolist())
    for blk in planted:
        t = blk * BLOCK + int(rng.integers(0, BLOCK))
        for kv in range(4):
            k[t, kv] = q[kv * 8: kv * 8 + 8].sum(axis=0)      # aligned with its 8 query heads
    ids, _ = msa.indexer(q, w, k, 40 * BLOCK - 1)
    assert ids.tolist() == planted + [39]


def test_gqa_head_mapping_and_relu():
    # a key planted in KV head 2 only matters to query heads 16..23
    rng = np.random.default_rng(6)
    q = _rand_fp8_values(rng, (32, 128))
    k = np.zeros((30 * BLOCK, 4, 128))
    w = np.zeros(32)
    w[16:24] = 1.0
    k[5 * BLOCK + 3, 2] = q[16:24].sum(axis=0)     # head group of KV head 2
    k[9 * BLOCK + 3, 1] = q[16:24].sum(axis=0) * 10  # wrong group: no effect
    k[12 * BLOCK + 3, 2] = -q[16:24].sum(axis=0) * 10  # negative logits: ReLU clips to 0
    s = msa.token_scores(q, w, k, 30 * BLOCK - 1)
    assert s[5 * BLOCK + 3] > 0
    assert s[9 * BLOCK + 3] == 0 and s[12 * BLOCK + 3] == 0
    ids, b = msa.indexer(q, w, k, 30 * BLOCK - 1)
    assert 5 in ids.tolist() and b[5] > 0 and b[12] == 0


def test_block_score_is_max_not_mean():
    # block 1: one spike token; block 2: every token moderately high (larger mean)
    s = np.zeros(20 * BLOCK)
    s[1 * BLOCK + 7] = 10.0
    s[2 * BLOCK: 3 * BLOCK] = 5.0
    b = msa.block_scores(s, 20 * BLOCK - 1)
    assert b[1] == 10.0 and b[2] == 5.0
    assert msa.select_blocks(b, 1).tolist() == [1, 19]


def test_causal_positions():
    rng = np.random.default_rng(7)
    q = _rand_fp8_values(rng, (32, 128))
    k = _rand_fp8_values(rng, (2500, 4, 128))
    w = rng.random(32)
    pos = 2400
    a, ba = msa.indexer(q, w, k, pos)
    k2 = k.copy()
    k2[pos + 1:] = 1000.0                 # tokens after pos must not matter
    b, bb = msa.indexer(q, w, k2, pos)
    assert np.array_equal(a, b) and np.array_equal(ba, bb)
    assert len(ba) == pos // BLOCK + 1


def _sdpa_fp64(q, k, v, scale):
    # q [Hq, D]; k, v [T, Hkv, D]; GQA by repeating KV heads
    g = q.shape[0] // k.shape[1]
    kk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, 0)   # [Hq, T, D]
    vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, 0)
    qq = torch.from_numpy(q)[:, None, :]                                 # [Hq, 1, D]
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
    return o[:, 0, :].numpy()


def test_sparse_equals_dense_equals_sdpa_when_all_blocks_fit():
    rng = np.random.default_rng(8)
    q = _rand_fp8_values(rng, (32, 128))
    k = _rand_fp8_values(rng, (17 * BLOCK, 4, 128))
    v = _rand_fp8_values(rng, (17 * BLOCK, 4, 128))
    w = rng.random(32)
    scale = 1 / np.sqrt(128)
    for pos in (0, 1, 127, 128, 1000, 17 * BLOCK - 1):
        ids, _ = msa.indexer(q, w, k, pos)
        sp = msa.sparse_attention(q, k, v, ids, pos, scale)
        de = msa.dense_attention(q, k, v, pos, scale)
        ref = _sdpa_fp64(q, k[: pos + 1], v[: pos + 1], scale)
        assert np.allclose(sp, ref, rtol=0, atol=1e-12)
        assert np.allclose(de, ref, rtol=0, atol=1e-12)


def test_sparse_differs_from_dense_when_blocks_dropped():
    rng = np.random.default_rng(9)
    q = _rand_fp8_values(rng, (32, 128))
    k = _rand_fp8_values(rng, (40 * BLOCK, 4, 128))
    v = _rand_fp8_values(rng, (40 * BLOCK, 4, 128))
    w = rng.random(32)
    pos = 40 * BLOCK - 1
    ids, _ = msa.indexer(q, w, k, pos)
    sp = msa.sparse_attention(q, k, v, ids, pos, 1 / np.sqrt(128))
    de = msa.dense_attention(q, k, v, pos, 1 / np.sqrt(128))
    assert np.abs(sp - de).max() > 1e-3


def test_attention_closed_forms():
    rng = np.random.default_rng(10)
    q = _rand_fp8_values(rng, (32, 128))
    v = _rand_fp8_values(rng, (300, 4, 128))
    k = _rand_fp8_values(rng, (300, 4, 128))
    o = msa.sparse_attention(q, k, v, np.array([0] + [-1] * 16), 0, 0.1)
    assert np.array_equal(o, np.repeat(v[0], 8, axis=0))        # one visible token
    kc = np.broadcast_to(k[:1], k.shape).copy()                 # identical keys -> mean of V
    ids = np.array([0, 1, 2] + [-1] * 14)
    o = msa.sparse_attention(q, kc, v, ids, 299, 0.1)
    assert np.allclose(o, np.repeat(v[:300].mean(axis=0), 8, axis=0), atol=1e-12)


def test_end_to_end_on_quantized_cache():
    # the indexer and attention run on FP8 values dequantised from the NVFP4 pool
    rng = np.random.default_rng(11)
    L = 25 * BLOCK + 37
    src = rng.standard_normal((L, 4, 128)).astype(np.float32)
    codes, scales = nvfp4.empty_pool(30, 4)
    bt = rng.permutation(30)[:26]
    slots = np.array([bt[t // BLOCK] * BLOCK + t % BLOCK for t in range(L)])
    nvfp4.write_cache(codes, scales, src, slots)
    gc, gs = nvfp4.gather_sequence(codes, scales, bt, L)
    _, khat = nvfp4.dequant_fp8(gc, gs)
    c, s = nvfp4.quantize(src)
    _, direct = nvfp4.dequant_fp8(c, s)
    assert np.array_equal(khat, direct)
    q = _rand_fp8_values(rng, (32, 128))
    ids, b = msa.indexer(q, rng.random(32), khat, L - 1)
    assert check_selection(b, ids) is None
    assert ids[-1] == 25 and len(set(ids.tolist())) == 17


def test_acceptance_rule_behaviour():
    b = np.linspace(1.0, 2.0, 40)
    ids = msa.select_blocks(b)
    assert check_selection(b, ids) is None
    bad = ids.copy()
    bad[0] = 0
    bad.sort()
    assert check_selection(b, bad) is not None
    # near tie between candidates 16 and 17: either may be picked
    b2 = np.arange(40, dtype=np.float64) + 100
    b2[22] = b2[23] * (1 + 1e-6)
    ids2 = msa.select_blocks(b2).tolist()
    assert check_selection(b2, np.array(ids2)) is None
    assert 22 in ids2 and 23 not in ids2
    alt = sorted([i for i in ids2[:-1] if i != 22] + [23]) + [39]
    assert check_selection(b2, np.array(alt)) is None          # the near-tied 17th is fine
    far = sorted([i for i in ids2[:-1] if i != 38] + [0]) + [39]
    assert check_selection(b2, np.array(far)) is not None      # a clear winner missing is not
