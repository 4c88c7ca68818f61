"""JoLT oracle: a plain, slow, float64 CPU implementation of what the
compressed-cache decode path computes.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The product path (the
HIP library and its Python binding) never imports, calls or links anything
here, and this package imports nothing from the product path.

Sources (web pages on JoLT; cited by title and section in every module):

* "A JoLT for the KV cache: Near-Lossless KV Cache Compression via Joint
  Rank-bit Allocation" -- the arXiv 2607.12550v4 summary on paperlayer.ai
  (Abstract, §1, §3 Method, §3.1, §4.4, §4.5, §5, App. E).  The authority.
* "Technische Samenvatting: Een JOLT voor de KV Cache" (gist.science, Dutch)
  and the French "Résumé Technique" on gist.science -- method summaries
  (partial Tucker / ST-HOSVD, JL-rotated residual, Lagrangian allocation).
* "JoLT: совместное распределение ранга и бит в KV-кэше" (sarnas.ru blog) --
  the KV-byte formula and in-kernel RoPE cos/sin from int32 positions.
* The hegai.media news piece on KV-cache compression -- the 70B byte figures.

Modules:

* ``accounting``  KV and compressed-cell byte counts.
* ``storage``     rounding to the stored factor dtype.
* ``tucker``      partial Tucker (ST-HOSVD) on the token and feature modes.
* ``rotation``    the seeded random orthogonal (JL) rotation.
* ``quant``       uniform b-bit quantiser and code packing.
* ``allocate``    the single-multiplier rank/bit allocator.
* ``compress``    the compressor pipeline (grouped cache -> stored cell).
* ``rope``        rotary position embedding at fp32 angles.
* ``attention``   decode attention over the decoded cache, and dense decode.

Parity status: every function is pinned by a CPU test against values the
pages print, closed forms, special cases that reduce to a library routine, or
brute force (see tests/test_oracle_*.py).  The allocator's choices on real
model caches and the pages' reconstruction errors on real models cannot be
reproduced without model weights: those comparisons are parity unpinned.
"""
