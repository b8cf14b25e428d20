"""Block splitter and ring schedules, pure Python (test infrastructure).

Used only to check invariants of the oracle (blockwise == one-shot, merge
order independence) and to pin the library's host-side planner.  It shares no
code with that planner.

Sources (pages cited by title and section):

* Ring Attention record (anthology-of-the-sota, Liu et al. 2023): every device
  keeps its query block and passes its K/V block to its neighbour each step, so
  rank r sees K/V blocks r, r-1, r-2, ... (mod P) in steps 0, 1, 2, ...
* TokenRing review (pith.science), "Core claim" and the Algorithm 1 major
  comment (paper section 3.2): K/V stays put, query blocks travel forward one
  hop per iteration and each partial (block_out, block_lse) goes back to the
  rank that owns those query rows.  Reading of the undefined ``step``: it is
  the 1-based iteration i, with every index taken mod N; at iteration i rank j
  computes Q_t against its own K/V with t = (j - i + 1) mod N.  So the owner t
  receives partials for K/V blocks t, t+1, ..., t+N-1 (ascending, mod N).
* Zigzag causal partition (TokenRing review, "If this is right" and the
  section 3.3.2 minor comment; no pseudo-code on the pages): the sequence is
  cut into 2P equal chunks and rank r holds chunks r and 2P-1-r, which gives
  every rank the same number of visible causal pairs.
"""

from __future__ import annotations

import itertools

import numpy as np

from .attention import attention
from .merge import merge_stable, merge_literal, merge_bshd

LAYOUTS = ("contig", "contig_causal", "zigzag_causal", "kv_sharded", "kv_sharded_causal")


def contiguous_shares(S: int, P: int):
    """Rank r owns token rows [r*S/P, (r+1)*S/P)."""
    if S % P:
        raise ValueError("S must be a multiple of P")
    n = S // P
    return [np.arange(r * n, (r + 1) * n, dtype=np.int64) for r in range(P)]


def zigzag_chunks(S: int, P: int):
    """Rank r owns chunks r and 2P-1-r of length S/(2P), in that local order."""
    if S % (2 * P):
        raise ValueError("S must be a multiple of 2P for the zigzag layout")
    c = S // (2 * P)
    chunk = lambda i: np.arange(i * c, (i + 1) * c, dtype=np.int64)
    return [np.concatenate([chunk(r), chunk(2 * P - 1 - r)]) for r in range(P)]


def rank_rows(S: int, P: int, layout: str):
    if layout in ("contig", "contig_causal"):
        return contiguous_shares(S, P)
    if layout == "zigzag_causal":
        return zigzag_chunks(S, P)
    raise ValueError(layout)


def ring_kv_order(r: int, P: int, order: str):
    """K/V ranks merged by owner r, step by step.

    ring:      (r - t) mod P  -- the K/V block arriving at step t.
    tokenring: (r + t) mod P  -- the partial for Q_r returned at iteration
                                 t+1 was computed on rank (r + t) mod P.
    """
    if order == "ring":
        return [(r - t) % P for t in range(P)]
    if order == "tokenring":
        return [(r + t) % P for t in range(P)]
    raise ValueError(order)


def tokenring_schedule(N: int):
    """Algorithm 1 under the reading above, as explicit tables.

    Returns a dict with, for rank j and iteration i = 1..N:
      compute[j][i-1] = owner t of the query block rank j attends to,
      send[j][i-1]    = owner of the partial sent at iteration i (the previous
                        iteration's), or None at i = 1,
      final_send[j]   = owner of the last partial, (j - N + 1) mod N,
      recv_q[j][i-1]  = True iff a query block arrives from rank j-1 (i > 1).
    """
    compute = [[(j - i + 1) % N for i in range(1, N + 1)] for j in range(N)]
    send = [[None if i == 1 else compute[j][i - 2] for i in range(1, N + 1)] for j in range(N)]
    final_send = [(j - N + 1) % N for j in range(N)]
    recv_q = [[i > 1 for i in range(1, N + 1)] for j in range(N)]
    return {"compute": compute, "send": send, "final_send": final_send, "recv_q": recv_q}


def visible_pairs_per_rank(S: int, P: int, layout: str):
    """Visible (query, key) pairs of each rank's rows, by direct counting."""
    rows = rank_rows(S, P, layout)
    causal = layout != "contig"
    if not causal:
        return [len(rr) * S for rr in rows]
    # Under the causal mask query position i sees keys 0..i: i+1 keys.
    return [int(np.sum(rr + 1)) for rr in rows]


def ring_blockwise(q, k, v, P: int, layout: str = "contig", order: str = "ring",
                   ranks=None, rule: str = "stable"):
    """Emulate the P-step ring on the CPU and return natural-order (out, lse).

    Every step, each rank attends its query rows to one K/V block (with the
    causal mask on global positions where the layout is causal) and folds the
    partial into its running pair with the sigma rule.  Rows of ranks not in
    ``ranks`` stay at the identity (0, -inf).

    layout: "contig" | "contig_causal" | "zigzag_causal" | "kv_sharded" |
      "kv_sharded_causal"
      ("kv_sharded": queries are not partitioned; K/V is cut into P contiguous
       blocks, each visited once -- the decode-style shape.  "kv_sharded_causal":
       the same, with the queries taken as the last Sq of the Sk positions and
       the causal mask applied on positions -- a prefill chunk or a decode step
       at the end of a sharded cache.)
    rule: "stable" (merge_stable) or "literal" (merge_literal; finite only).
    """
    B, Sq, Hq, d = q.shape
    Sk = k.shape[1]
    merge = merge_stable if rule == "stable" else merge_literal
    out = np.zeros((B, Sq, Hq, d), dtype=np.float64)
    lse = np.full((B, Hq, Sq), -np.inf, dtype=np.float64)

    q_shift = 0
    if layout in ("kv_sharded", "kv_sharded_causal"):
        q_rows = [np.arange(Sq, dtype=np.int64)]
        kv_rows = contiguous_shares(Sk, P)
        owners = [0]
        causal = layout == "kv_sharded_causal"
        if causal:
            if Sq > Sk:
                raise ValueError("kv_sharded_causal needs Sq <= Sk")
            q_shift = Sk - Sq     # query row i sits at position Sk - Sq + i
    else:
        if Sq != Sk:
            raise ValueError("ring layouts need Sq == Sk")
        q_rows = rank_rows(Sq, P, layout)
        kv_rows = q_rows
        owners = list(range(P)) if ranks is None else list(ranks)
        causal = layout != "contig"

    for r in owners:
        rr = q_rows[r]
        run_out = np.zeros((B, len(rr), Hq, d))
        run_lse = np.full((B, Hq, len(rr)), -np.inf)
        kv_order = ring_kv_order(r if not layout.startswith("kv_sharded") else 0, P, order)
        for s in kv_order:
            kk = kv_rows[s]
            bo, bl = attention(q[:, rr], k[:, kk], v[:, kk], causal=causal,
                               q_pos=rr + q_shift, k_pos=kk)
            if rule == "literal" and not np.all(np.isfinite(run_lse)):
                # The printed rule is undefined at lse = -inf; the first
                # block is taken as is (the rule's limit there).
                run_out, run_lse = bo, bl
            else:
                run_out, run_lse = merge_bshd(run_out, run_lse, bo, bl, merge)
        out[:, rr] = run_out
        lse[:, :, rr] = run_lse
    return out, lse


def all_orders(P: int):
    """Every permutation of K/V block visits (for order-independence tests)."""
    return list(itertools.permutations(range(P)))
