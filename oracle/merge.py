"""The sigma / ln-sigma merge rule in fp64 (test infrastructure).

Source: TokenRing review (pith.science), "What carries the argument" (paper
section 3.1).  A running pair (out, lse) for a set of query rows absorbs a
partial (block_out, block_lse) computed against one more K/V block by

    out <- out - sigma(block_lse - lse) * (out - block_out)
    lse <- lse - ln sigma(lse - block_lse)

with sigma(x) = 1 / (1 + exp(-x)).  Readings (the pages are silent on them):

* Both right-hand sides use the *old* lse (simultaneous assignment): the rule
  is the two-term log-sum-exp combination, and only that order makes it so.
* lse is a natural logarithm ("ln" in the rule).
* The running pair starts at (out, lse) = (0, -inf), the rule's identity.  At
  lse = -inf the literal second line is -inf + inf; ``merge_stable`` evaluates
  the same quantity as max(lse, blse) + ln(1 + exp(-|lse - blse|)), which is
  algebraically identical wherever the literal form is finite.
"""

from __future__ import annotations

import numpy as np


def sigmoid(x):
    """sigma(x) = 1 / (1 + exp(-x)), evaluated without overflow warnings."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def merge_literal(out, lse, block_out, block_lse):
    """The rule exactly as printed.  Finite lse values only.

    out, block_out: [..., d];  lse, block_lse: [...] (same leading shape).
    Returns the new (out, lse); the inputs are not modified.
    """
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    block_out = np.asarray(block_out, dtype=np.float64)
    block_lse = np.asarray(block_lse, dtype=np.float64)
    w = sigmoid(block_lse - lse)
    new_out = out - w[..., None] * (out - block_out)
    new_lse = lse - np.log(sigmoid(lse - block_lse))
    return new_out, new_lse


def merge_stable(out, lse, block_out, block_lse):
    """Same rule, evaluated so that -inf (an empty partial) is the identity.

    Cases: block_lse = -inf keeps (out, lse); lse = -inf takes the block;
    otherwise sigma(block_lse - lse) weights the block and the new lse is
    max + ln(1 + exp(-|difference|)).
    """
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    block_out = np.asarray(block_out, dtype=np.float64)
    block_lse = np.asarray(block_lse, dtype=np.float64)
    lse_b, blse_b = np.broadcast_arrays(lse, block_lse)
    block_empty = np.isneginf(blse_b)
    run_empty = np.isneginf(lse_b) & ~block_empty
    both = ~block_empty & ~run_empty

    with np.errstate(invalid="ignore"):
        diff = np.where(both, blse_b - lse_b, 0.0)
    w = np.where(run_empty, 1.0, np.where(block_empty, 0.0, sigmoid(diff)))
    new_out = out - w[..., None] * (out - block_out)
    hi = np.maximum(lse_b, blse_b)
    new_lse = np.where(
        both, hi + np.log1p(np.exp(-np.abs(diff))),
        np.where(block_empty, lse_b, blse_b))
    # Rows where the running pair is empty take the block verbatim (avoids
    # 0 - 1*(0 - x) rounding noise; it is exact anyway in IEEE arithmetic).
    new_out = np.where(run_empty[..., None], block_out, new_out)
    return new_out, new_lse


def merge_bshd(out, lse, block_out, block_lse, rule=merge_stable):
    """Apply ``rule`` to tensors in the attention layout.

    out, block_out: [B, S, H, d];  lse, block_lse: [B, H, S] (the layout the
    attention oracle returns).  The rule itself is row-wise.
    """
    o, l = rule(out, np.swapaxes(lse, 1, 2), block_out, np.swapaxes(block_lse, 1, 2))
    return o, np.ascontiguousarray(np.swapaxes(l, 1, 2))
