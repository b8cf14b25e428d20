"""CPU oracle for exact blockwise (ring) attention -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct fp64 reference that the HIP
path is checked against.  It is test infrastructure: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``ring_blockwise_softmax_amd``) never imports,
calls or links anything here, and nothing here imports the product path.  The
two sides share no code; only the seeded input generators (a module of their
own that holds none of the method's arithmetic) feed both.

What it computes (sources are the pages, cited by title and section):

* ``attention``      -- one-shot softmax attention with its row log-sum-exp.
  The method is exact: the Ring Attention record (anthology-of-the-sota,
  "Liu et al. 2023", the paragraph on the claim) says the ring reaches the same
  attention without approximation, and the TokenRing review (pith.science,
  "What carries the argument"; paper section 3.1) says the merge rule stitches
  the partials into exact attention.  So the reference *is* the plain
  definition, not a blockwise algorithm.
* ``merge_literal`` / ``merge_stable`` -- the sigma / ln-sigma update rule of
  the TokenRing review, "What carries the argument" (paper section 3.1).
* ``blockwise``      -- a pure-Python block splitter and ring schedules (Ring
  Attention's K/V rotation; TokenRing's Q-forward / partial-back order; the
  zigzag causal partition of the TokenRing review, "If this is right" and the
  section 3.3.2 minor comment), used only to check invariants.

Pins (each in ``tests/``, run with ``-m "not gpu"``): brute force with scalar
``math.fsum`` loops on tiny inputs, closed forms (uniform weights when Q = 0,
constant V per K/V head, one-hot V, single key), merge-rule algebra (identity,
self-merge, order independence, associativity), blockwise == one-shot, and a
cross-check of ``out`` against torch's CPU fp64 scaled-dot-product attention.
No function here is "parity unpinned".
"""

from .attention import attention, kv_head_of
from .merge import merge_literal, merge_stable, merge_bshd, sigmoid
from .blockwise import (
    contiguous_shares,
    zigzag_chunks,
    ring_kv_order,
    tokenring_schedule,
    ring_blockwise,
    visible_pairs_per_rank,
)

__all__ = [
    "attention",
    "kv_head_of",
    "merge_literal",
    "merge_stable",
    "merge_bshd",
    "sigmoid",
    "contiguous_shares",
    "zigzag_chunks",
    "ring_kv_order",
    "tokenring_schedule",
    "ring_blockwise",
    "visible_pairs_per_rank",
]
