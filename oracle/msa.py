"""MiniMax-style sparse attention decode, one query token at a time
(oracle; test infrastructure).

The pages (MiniMax-M3.1-Flash serving summary, yuxiaoba.github.io, section
"Sparse attention still scans an index"): KV is organised in 128-token
blocks; a lightweight indexer scores the context, selects 16 blocks and also
keeps the most recent block; exact attention then runs over those roughly
2,048 keys only, which is not the same as dense attention. Queries are FP8
and the cache is converted to FP8 before the products (MiniMax-M3.1-Flash
lands in vLLM on day one, third paragraph), so every operand here is an FP8
value held in float64 and all arithmetic is float64.

Positions: a sequence of length L holds tokens 0..L-1, including its Q query
tokens, whose keys are already in the cache; query token i (0-based) sits at
pos = L - Q + i and sees tokens t <= pos (causal within a speculative draft).
Its visible blocks are 0..nb-1 with nb = pos // 128 + 1; block nb-1 is the
most recent one.

Readings where the pages are silent (parity of the first two is unpinned by
the pages; the oracle's implementation of them is pinned by planted-block
and invariance tests):
  token score   S(t) = sum_h w_h * max(0, q_h . K(t, h // G)), G = Hq / H_idx
  block score   B(i) = max of S(t) over the block's visible tokens
  selection     the 16 best of blocks 0..nb-2 by (score descending, block
                index ascending) plus block nb-1, listed in ascending order;
                every block when nb <= 17; -1 padding to 17 entries
  attention     softmax(scale * q_h . K(t)) over the selected visible tokens,
                weights applied to V(t); query head h reads KV head h // G
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


def num_visible_blocks(pos: int, block: int = BLOCK) -> int:
    return pos // block + 1


def token_scores(q, w, khat, pos):
    """S(t) for t = 0..pos.

    q    float64 [Hq, D]   index-query values (FP8-exact)
    w    float64 [Hq]      head weights
    khat float64 [>=pos+1, H_idx, D] index-key values (FP8-exact)
    """
    q = np.asarray(q, dtype=np.float64)
    hq, hidx = q.shape[0], khat.shape[1]
    g = hq // hidx
    k = np.asarray(khat[: pos + 1], dtype=np.float64)
    logits = np.empty((pos + 1, hq))
    for h in range(hq):
        logits[:, h] = k[:, h // g, :] @ q[h]
    return (np.maximum(logits, 0.0) * np.asarray(w, dtype=np.float64)[None, :]).sum(axis=1)


def block_scores(s, pos, block: int = BLOCK):
    """B(i) = max of S over block i's visible tokens, i = 0..nb-1."""
    nb = num_visible_blocks(pos, block)
    return np.array([np.max(s[i * block: min((i + 1) * block, pos + 1)]) for i in range(nb)])


def select_blocks(bscores, topk: int = 16):
    """Top-`topk` of the non-recent blocks plus the recent one, ascending, -1 padded."""
    nb = len(bscores)
    out = np.full(topk + 1, -1, dtype=np.int32)
    if nb <= topk + 1:
        out[:nb] = np.arange(nb)
        return out
    cand = np.arange(nb - 1)
    order = np.lexsort((cand, -np.asarray(bscores[: nb - 1], dtype=np.float64)))
    out[:topk] = np.sort(cand[order[:topk]])
    out[topk] = nb - 1
    return out


def indexer(q, w, khat, pos, topk: int = 16, block: int = BLOCK):
    """(selected block ids [topk+1], block scores [nb]) for one query token."""
    b = block_scores(token_scores(q, w, khat, pos), pos, block)
    return select_blocks(b, topk), b


def _attend(q, khat, vhat, tokens, scale):
    q = np.asarray(q, dtype=np.float64)
    hq, hkv = q.shape[0], khat.shape[1]
    g = hq // hkv
    out = np.empty((hq, q.shape[1]))
    for h in range(hq):
        z = (khat[tokens, h // g, :] @ q[h]) * scale
        p = np.exp(z - z.max())
        out[h] = (p @ vhat[tokens, h // g, :]) / p.sum()
    return out


def selected_tokens(ids, pos, block: int = BLOCK):
    parts = [np.arange(b * block, min((b + 1) * block, pos + 1)) for b in ids if b >= 0]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def sparse_attention(q, khat, vhat, ids, pos, scale, block: int = BLOCK):
    """Exact attention of one query token over the visible tokens of blocks `ids`.

    q [Hq, D]; khat, vhat [>=pos+1, Hkv, D] (FP8-exact float64) -> [Hq, D].
    """
    return _attend(q, khat, vhat, selected_tokens(ids, pos, block), scale)


def dense_attention(q, khat, vhat, pos, scale):
    """Attention over every token 0..pos (the reference the sparse path is not
    equal to once a block is left out)."""
    return _attend(q, khat, vhat, np.arange(pos + 1), scale)
