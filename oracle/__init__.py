"""Oracle for the Kimi Delta Attention (KDA) hot path.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg are the only callers. The product path (the HIP library and its Python
binding) never imports, links or executes anything here, and nothing here imports the product.

Source of every formula: the Kimi K3 reading notes (liuzhao09.github.io/papers/kimi-k3.html),
section 2.2 "Hybrid KDA-MLA and Block AttnRes" (recurrence equation, cumulative-decay equation,
chunk equation, decay lower-bound equation) and section 2.5 (affine pair of a segment).

Modules
  native     -- plain C fp64 token loop (``kda_oracle.c``), OpenMP over (lane, column block)
  recurrence -- the same recurrence in numpy fp64, vectorised over lanes, plus the explicit
                product form of the transition matrices
  chunked    -- numpy fp64 chunkwise form (UT transform, derived pieces noted in the module)
  exact      -- exact rational arithmetic (``fractions``) for tiny inputs

Parity status: every function here is pinned by ``tests/test_oracle_*.py`` to facts fixed by
the pages or by mathematics (exact rationals, closed forms, invariants, a worked example).
"""
