"""The decode workloads: shapes, seeds, lengths and block tables.

All five share one head layout: 4 KV heads and 4 index-key heads of
dimension 128, 32 FP8 query heads (8 per KV head), 128-token pages/blocks,
top-16 + the most recent block.

Block tables are int32 [B, max_blocks]; entries past a sequence's last block
are -1 and are never read.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import synth


@dataclass
class Workload:
    name: str
    seed: int
    seq_lens: list           # per sequence; includes the query tokens
    q_per_seq: int
    num_pages: int
    block_table: np.ndarray  # int32 [B, max_blocks]
    outliers: bool = False
    num_kv_heads: int = 4
    num_idx_heads: int = 4
    num_q_heads: int = 32
    head_dim: int = 128
    block_tokens: int = 128
    topk: int = 16
    description: str = ""
    _outlier_cache: dict = field(default_factory=dict, repr=False)

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def num_q_tokens(self) -> int:
        return self.num_seqs * self.q_per_seq

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    def blocks_of(self, b: int) -> int:
        return (int(self.seq_lens[b]) + self.block_tokens - 1) // self.block_tokens

    def pages_in_use(self) -> np.ndarray:
        ids = [self.block_table[b, : self.blocks_of(b)] for b in range(self.num_seqs)]
        return np.unique(np.concatenate(ids)).astype(np.int64)

    def num_heads_of(self, stream: int) -> int:
        return self.num_idx_heads if stream == synth.STREAM_IDX else self.num_kv_heads

    def outlier_mask(self, stream: int):
        """bool [H, D]: round(0.05 * D) channels per head scaled x8, or None."""
        if not self.outliers:
            return None
        if stream not in self._outlier_cache:
            h = self.num_heads_of(stream)
            n = int(round(0.05 * self.head_dim))
            rng = np.random.default_rng([self.seed, 100 + stream])
            m = np.zeros((h, self.head_dim), dtype=bool)
            for i in range(h):
                m[i, rng.choice(self.head_dim, n, replace=False)] = True
            self._outlier_cache[stream] = torch.from_numpy(m)
        return self._outlier_cache[stream]

    def sources(self, stream: int, pages, device="cpu") -> torch.Tensor:
        """fp32 sources [len(pages)*128, H, D] for the given physical pages."""
        pages = torch.as_tensor(np.asarray(pages, dtype=np.int64), device=device)
        return synth.page_sources(self.seed, stream, pages, self.num_heads_of(stream),
                                  self.head_dim, self.block_tokens,
                                  self.outlier_mask(stream))

    def q_idx(self) -> torch.Tensor:
        return synth.query_fp8(self.seed, synth.STREAM_QIDX, self.num_q_tokens, self.num_q_heads,
                               self.head_dim)

    def q_attn(self) -> torch.Tensor:
        return synth.query_fp8(self.seed, synth.STREAM_QATTN, self.num_q_tokens,
                               self.num_q_heads, self.head_dim)

    def weights(self) -> torch.Tensor:
        return synth.head_weights(self.seed, self.num_q_tokens, self.num_q_heads)

    def positions(self, b: int) -> list:
        L = int(self.seq_lens[b])
        return [L - self.q_per_seq + i for i in range(self.q_per_seq)]


def _identity_table(nblocks: list, width: int | None = None) -> np.ndarray:
    width = width or max(nblocks)
    bt = np.full((len(nblocks), width), -1, dtype=np.int32)
    p = 0
    for b, n in enumerate(nblocks):
        bt[b, :n] = np.arange(p, p + n, dtype=np.int32)
        p += n
    return bt


def _cfg_tiny_4k() -> Workload:
    return Workload("tiny_decode_1x4k", 0, [4096], 1, 32, _identity_table([32]),
                    description="batch 1, 4,096-token context (32 blocks), 1 query token")


def _cfg_batch_32x32k() -> Workload:
    B, nb, pool = 32, 256, 8192
    perm = np.random.default_rng([1, 200]).permutation(pool).astype(np.int32)
    return Workload("batch_decode_32x32k_outliers", 1, [32768] * B, 1, pool,
                    perm.reshape(B, nb), outliers=True,
                    description="32 x 32,768 tokens, 1 query token, page-permuted pool, "
                                "5% outlier channels x8")


def _cfg_long_8x256k() -> Workload:
    B, nb = 8, 2048
    return Workload("long_context_8x256k", 2, [262144] * B, 1, B * nb,
                    _identity_table([nb] * B),
                    description="8 x 262,144 tokens (2,048 blocks), 1 query token")


def _cfg_spec_16x64k() -> Workload:
    B, nb = 16, 512
    return Workload("spec_verify_16x64k_q8", 3, [65536] * B, 8, B * nb,
                    _identity_table([nb] * B),
                    description="16 x 65,536 tokens, 8 query tokens per sequence "
                                "(7 draft + 1), causal within the draft")


def _cfg_ragged_45() -> Workload:
    rng = np.random.default_rng(7)
    lens = (np.round(rng.uniform(30720, 215040, 45) / 128).astype(np.int64) * 128).tolist()
    shared = 16384 // 128
    nbs = [L // 128 for L in lens]
    bt = np.full((45, max(nbs)), -1, dtype=np.int32)
    p = shared
    for b, n in enumerate(nbs):
        bt[b, :shared] = np.arange(shared, dtype=np.int32)
        bt[b, shared:n] = np.arange(p, p + n - shared, dtype=np.int32)
        p += n - shared
    return Workload("ragged_45req_shared_prefix", 7, lens, 1, p, bt,
                    description="45 requests, lengths U[30,720, 215,040] rounded to 128, "
                                "first 16,384 tokens shared (same physical pages)")


CONFIGS = {
    0: _cfg_tiny_4k,
    1: _cfg_batch_32x32k,
    2: _cfg_long_8x256k,
    3: _cfg_spec_16x64k,
    4: _cfg_ragged_45,
}


def get_config(i: int) -> Workload:
    return CONFIGS[i]()


def tiny_config(seq_lens, q_per_seq=1, seed=11, spare_pages=5, permute=True,
                outliers=False, name="tiny", shared=()) -> Workload:
    """Small ragged workload over a permuted pool with spare (unused) pages.
    shared: (member sequences, blocks) pairs; the members' first `blocks`
    logical blocks are mapped to the first member's pages (a common prefix;
    the pages they had become spare)."""
    nbs = [(L + 127) // 128 for L in seq_lens]
    total = sum(nbs) + spare_pages
    bt = np.full((len(seq_lens), max(nbs)), -1, dtype=np.int32)
    order = (np.random.default_rng([seed, 300]).permutation(total) if permute
             else np.arange(total)).astype(np.int32)
    p = 0
    for b, n in enumerate(nbs):
        bt[b, :n] = order[p:p + n]
        p += n
    for members, blocks in shared:
        for b in members[1:]:
            n = min(blocks, nbs[b], nbs[members[0]])
            bt[b, :n] = bt[members[0], :n]
    return Workload(name, seed, list(seq_lens), q_per_seq, total, bt, outliers=outliers)
