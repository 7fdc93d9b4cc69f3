"""Radial-attention oracle: plain, slow, obviously correct CPU reference.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the C-ABI library or
its Python binding) imports, calls or links anything in this package.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.

Sources cited in this package (abbreviations used in docstrings):

* "review"   -- the jaehun.me paper review *Radial Attention: O(n log n) Sparse
  Attention with Energy Decay for Long Video Generation* (Prompt 1.3.1 walks
  through the method step by step; the toy example uses f=4, s=9).  Section
  names in brackets (paper §3, §4.2, Eq.4, Fig.5 ...) are the paper's own
  numbering as the review quotes it.
* "rebuttal" -- the paperhub.cn author-response page *Radial Attention:
  O(n log n) Sparse Attention for Long Video Generation* (ablations of the
  attention sink, central-band width and band width scale).
* "abstract" -- the paper abstract (chatpaper.ai / scholarfeed pages).

Modules:

* ``oracle.mask``      -- band table, token predicate, brute-force token mask,
  closed-form pair count, tile cover (CSR/CSC) by a per-(query token, key
  frame) interval sweep.
* ``oracle.attention`` -- masked softmax attention forward (O, LSE) and its
  gradient (dQ, dK, dV) in float64 numpy.

Parity status: every function is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` against the review's worked example, closed forms,
brute force or a library routine (torch SDPA / autograd in float64).  The
sub-1-width sampling rule (``band`` with w == 0) is pinned by the
power-of-two special case s == 1 and, read off the brute-force mask at
frame sizes where ceil and floor of 2^r / s differ, by its structure (empty
or diagonal blocks) and the band density bound (2^-r / 2, 2^-r]; the pages
give no worked numbers for it, so the exact period inside that bound is
parity unpinned.  ``attention.bwd_dkdv_tile`` / ``row_stats`` (per key tile)
and ``fwd_rows`` / ``dq_rows`` (per query row set), and their token-mask
counterparts ``dkdv_masked_keys`` / ``row_stats_masked``, are pinned against
the whole-head functions and torch float64 autograd.
"""

from . import mask, attention  # noqa: F401
