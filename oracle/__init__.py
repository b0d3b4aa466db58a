"""Plain float64 CPU oracle for draft-tree verification through Gated DeltaNet layers.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import or run anything in this package. The product path (the HIP
library and its Python binding) never calls it and shares no code with it: no kernels,
helpers, tables or pre/post-processing. Inputs come from the seeded generators, which hold
none of the method's arithmetic.

Sources (cited by page title and section):
  [SpecLA guide]  "Lucebox SpecLA and Gated DeltaNet state-resident verification" (nxbn.cn
                  guide on linear-attention speculative decoding), sections "Why speculative
                  decoding is harder for linear-attention models", mechanisms 1-4 (state-
                  resident verification, HLD chains and waves, accepted-factor banks,
                  deferred fused commit) and "How correctness is guaranteed".
  [DFlash README] "Luce DFlash server README", section "How it works" (DDTree tree verify,
                  per-step rollback, tree-aware conv gather) and "Architecture note".

Modules:
  gdn    -- the gated delta rule along every root-to-node path; factors; commit by replay;
            two independent re-formulations (DFS state stack, tree-masked UT closed form).
  conv   -- tree-aware causal depthwise conv and the committed conv window.
  hld    -- heavy-light chain schedule (iterative and recursive formulations).
  banks  -- factor-bank compaction and role/pending bookkeeping.
  prologue -- conv -> SiLU -> unit-length q/k prologue feeding the tree verify (the reading
            of the q/k/v wiring the pages leave open, stated in its header).
  ddtree -- best-first draft-tree builder with budget, tau pruning and chain pre-seed.

Every function is pinned by tests/test_oracle_*.py against closed forms, invariants,
brute force, library routines of the plain definitions, or the hand-worked schedule and
draft-tree examples under tests/golden/. None is "parity unpinned".
"""
from . import banks, conv, gdn, hld  # noqa: F401
