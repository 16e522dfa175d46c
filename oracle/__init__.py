"""CPU oracle for draft branch attention under context parallelism.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package. The product path (the HIP library and its Python binding) never
imports, calls or links anything here, and this package imports nothing from
the product path.

What it computes, and where that is stated (page "paper.rainbus.top" = the
rainbus analysis of arXiv:2609.07108; page "ai.info" = the ai.info summary):

* ``pack``: the packed, load-balanced zigzag split of variable-length
  sequences over C context-parallel ranks (rainbus analysis, background
  section on context parallelism: each rank holds a head chunk and a tail
  chunk of the sequence; method steps, step two: C ranks hold N/C tokens each)
  and the anchor -> branch index (ai.info, Key Contributions 1: the branch part
  stays on the rank that owns the branch's anchor).
* ``attn``: dense masked softmax attention over the visible key set of every
  query row (ai.info, Methodology: a branch query sees the causal prefix of the
  main sequence plus its own branch-local keys; the split form is
  mathematically equal to the full attention), its closed-form backward, and
  the split form itself: per-ring-step partials and the branch-local partial
  merged by the online-softmax rule (rainbus analysis, core method, Eq. 2).

Numerics: float64 or float32 (``dtype`` argument), NumPy only; matrix
products use ``numpy.matmul``. Every function states the passage it follows.
Parity status of each function is listed in the module docstrings of
``pack`` and ``attn``; all of them are pinned by ``tests/test_oracle_*.py``.
"""

from . import pack, attn  # noqa: F401
