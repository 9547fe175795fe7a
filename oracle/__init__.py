"""fp64 CPU oracle for the chunkwise GDN-core prefill (dense and SparseGDN).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import anything from this package.  The HIP
library never calls it, and it shares no code, header, table or constant with
the HIP sources.

Source of truth: the web page "SparseGDN: Chunk Sparse in Linear Attention：
中文研读笔记" (reading notes of arXiv 2610.41420v1).  Citations below give the
paper section and equation as that page prints them, e.g. "Sec. 2.3, Eq. (8)".
Equation numbers follow the page's own grouping: (1)-(4) dense prefill,
(5)-(8) local Delta system and block-adjacent inverse, (9)-(10) tail score and
rank key, (11)-(12) lifetime, visibility and upgrade gain, (13)-(14) tier
budgets and split score, (15)-(16) deferred W and CSR events, (17)-(21)
event-sparse propagation, (22)-(25) two-chunk mapped output.

Modules
  gdn      dense operator: token recurrence, decay prefix, local Delta system,
           exact and block-adjacent solves, chunk form (Eqs. 1-8)
  detfp    fixed-order fp64 helpers that make selector decisions reproducible
  selector tail score, gate energy, tier budgets, dynamic selector, CSR
           event layout (Eqs. 9-16)
  sparse   deferred W, event-sparse H, two-chunk grouped O, end-to-end sparse
           prefill (Eqs. 15, 17-25)

Pins: every function is checked in ``tests/test_oracle_*.py`` against closed
forms, special cases, library routines, brute force or counts printed on the
page.  The selector's decisions on random data have no printed worked example
on the page; they are pinned by crafted inputs with hand-derived answers and by
invariants, and the end-to-end sparse outputs are pinned through the
all-events-kept fixed point and the Eq. (25) identity.
"""

from . import detfp, gdn, selector, sparse  # noqa: F401
