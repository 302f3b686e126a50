"""Oracle for the FlashAttention forward pass: plain, slow, CPU-only, float64.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this package: only the test suite, the smoke check and the CPU-baseline leg of
the benchmark use it. It shares no code with the HIP library; both sides are fed
by the seeded input generators in ``fa_workloads`` and nothing else.

Sources (the three web pages on tiled exact attention), cited by tag below:

* P1 -- "FlashAttention分块计算优化Transformer显存效率" (intelliparadigm.com):
  §1.1 standard vs. tiled computation and its loop skeleton, §1.2 the on-chip
  (SRAM) budget table, §2.1 the HBM access table, §2.2 causal block skipping
  and its N=8, B=2 figure, §3.2 the online-softmax update.
* P2 -- "14. FlashAttention Memory Model | FlashAttention 显存模型"
  (datawhalechina llm-algo-leetcode): Q1 score-matrix bytes, Q2 tile counts
  and working set, Q3 tile trade-off and materialisation ratio.
* P3 -- "Flash Attention 原理" (note.lovescie.com): the classic tiled method's
  six transfers vs. two, the blocked-softmax worked example on [1,2,3,4], the
  two pillars (tiling, recomputation).

Modules:

* ``attention``  -- ``attention_ref`` (the plain definition, S and P
  materialised), ``tiled_ref`` (the pages' block algorithm with the online
  softmax), ``brute_ref`` (scalar pure-Python loops), ``attention_probs``.
* ``blocks``     -- ``block_counts`` (tile classes of a causal/ragged launch),
  ``causal_figure`` (the P1 §2.2 glyph grid), ``traffic`` (the P1 §2.1 HBM
  model).
* ``memory``     -- the P2 memory-model helpers and the P1 §1.2 budget rows.
* ``merge``      -- the P3 blocked-softmax merge on a vector.
* ``backward``   -- ``attention_bwd_ref`` (dQ, dK, dV of the forward's
  definition by the chain rule, P materialised; the gradients the P3
  recomputation pillar rebuilds tile by tile), ``attention_bwd_sampled``
  (the same at chosen rows of one long head, query rows taken in chunks)
  and ``brute_bwd_ref`` (scalar loops); pinned by finite differences of
  ``attention_ref``.

Every function here is pinned by tests against values the pages print, closed
forms, invariants, a library routine, or brute force; none is "parity
unpinned".
"""

from .attention import attention_ref, attention_probs, tiled_ref, brute_ref
from .blocks import block_counts, block_pattern, causal_figure, traffic
from .memory import (score_bytes, tiles_1d, score_tiles, score_tile_bytes,
                     working_set_bytes, tile_tradeoff, materialization_ratio,
                     sram_budget, sram_formula_as_printed)
from .merge import blocked_softmax
from .backward import attention_bwd_ref, attention_bwd_sampled, brute_bwd_ref

__all__ = [
    "attention_ref", "attention_probs", "tiled_ref", "brute_ref",
    "block_counts", "block_pattern", "causal_figure", "traffic",
    "score_bytes", "tiles_1d", "score_tiles", "score_tile_bytes",
    "working_set_bytes", "tile_tradeoff", "materialization_ratio",
    "sram_budget", "sram_formula_as_printed", "blocked_softmax",
    "attention_bwd_ref", "attention_bwd_sampled", "brute_bwd_ref",
]
