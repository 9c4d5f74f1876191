"""Plain CPU oracle for MSA decode over an NVFP4 paged KV cache.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product (the HIP library and
its Python binding) never calls it, and this package imports nothing from the
product. It is written in NumPy, in fp64 wherever arithmetic is involved, and
follows the pages step by step with no blocking, fusion or reordering.

Modules
  formats    E4M3 and E2M1 element formats (decode, exact nearest-even encode)
  nvfp4      NVFP4 quantisation of 16-element groups, dequantisation to FP8,
             and the paged pool layout (byte counts, scatter, gather)
  msa        the indexer (token scores, block scores, top-16 + recent block)
             and exact attention over the selected blocks, plus dense attention
  acceptance the acceptance rules used to compare another implementation
             with this oracle
  insert     the cache-insertion path after the QKV projection (optional
             RMSNorm, RoPE, NVFP4 insert of K / V / index keys, FP8 queries)

Parity status (see each function's docstring for its pin):
  formats, nvfp4       pinned (library casts, closed forms, page byte counts)
  msa.select_blocks    pinned (brute force, invariants, page block counts)
  msa.sparse_attention pinned (library special case, closed forms)
  msa.token_scores / msa.block_scores: the pages say only that a lightweight
      indexer scores context per 128-token block; the score function
      sum_h w_h * ReLU(q_h . k) and the max over a block's tokens are this
      build's reading. The implementation of that reading is pinned by
      planted-block and invariance tests, but the reading itself is
      parity unpinned by the pages.
  insert               pinned (bf16 against torch, closed-form RMSNorm and RoPE
      cases, RoPE as a complex rotation, segment placement); which heads are
      normalised, the rotate-half pairing and the angle formula are this
      build's reading of "normalization, RoPE" on the pages.
"""
from . import formats, nvfp4, msa, acceptance, insert  # noqa: F401
