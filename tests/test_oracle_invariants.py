"""Pin the oracle's merge rule and ring emulation against algebra and invariants.

* The sigma rule of the TokenRing review ("What carries the argument"; paper
  section 3.1) is the two-term log-sum-exp combination: with weights
  a = e^lse, b = e^block_lse the new pair is ((a out + b bout)/(a+b),
  ln(a+b)).  Checked against that weighted form computed with scalar math.
* Exactness (Ring Attention record; TokenRing review, "Assumptions"): merging
  the partials of any split of the keys reproduces one-shot attention.
* Consequences: order independence, associativity, identity (0, -inf),
  self-merge adds ln 2, stable == literal wherever the literal is finite.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import attention, merge_literal, merge_stable, merge_bshd
from oracle.blockwise import (ring_blockwise, tokenring_schedule, ring_kv_order,
                              zigzag_chunks, visible_pairs_per_rank)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def _partials(q, k, v, splits, causal=False):
    """Block partials of one-shot attention over a partition of the keys."""
    parts = []
    for kk in splits:
        parts.append(attention(q, k[:, kk], v[:, kk], causal=causal,
                               q_pos=np.arange(q.shape[1]), k_pos=kk))
    return parts


def _fold(parts, rule):
    out = np.zeros_like(parts[0][0])
    lse = np.full_like(parts[0][1], -np.inf)
    for bo, bl in parts:
        if rule is merge_literal and np.all(np.isneginf(lse)):
            out, lse = bo, bl
        else:
            out, lse = merge_bshd(out, lse, bo, bl, rule)
    return out, lse


def _random_partition(rng, n, P):
    perm = rng.permutation(n)
    cuts = np.sort(rng.choice(np.arange(1, n), size=P - 1, replace=False)) if P > 1 else []
    return [np.sort(x) for x in np.split(perm, cuts)]


def test_merge_equals_weighted_logsumexp_scalar():
    rng = np.random.default_rng(0)
    for _ in range(200):
        d = 3
        o1, o2 = rng.standard_normal(d), rng.standard_normal(d)
        l1, l2 = rng.uniform(-30, 30), rng.uniform(-30, 30)
        # Scalar reference: weights e^l1, e^l2 shifted by their max.
        mx = max(l1, l2)
        a, b = math.exp(l1 - mx), math.exp(l2 - mx)
        ref_lse = mx + math.log(a + b)
        ref_out = [(a * o1[t] + b * o2[t]) / (a + b) for t in range(d)]
        for rule in (merge_literal, merge_stable):
            o, l = rule(o1[None], np.array([l1]), o2[None], np.array([l2]))
            assert abs(l[0] - ref_lse) < 1e-12
            assert np.max(np.abs(o[0] - ref_out)) < 1e-12


def test_golden_merge_cases():
    with open(os.path.join(GOLDEN, "merge_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        lse = np.array([float(c["lse"])])
        blse = np.array([float(c["block_lse"])])
        o, l = merge_stable(np.array([c["out"]]), lse, np.array([c["block_out"]]), blse)
        assert np.allclose(o[0], c["new_out"], rtol=0, atol=1e-14), c["name"]
        exp_l = float(c["new_lse"])
        if math.isinf(exp_l):
            assert l[0] == exp_l, c["name"]
        else:
            assert abs(l[0] - exp_l) < 1e-14, c["name"]
        if all(math.isfinite(float(c[x])) for x in ("lse", "block_lse")):
            o2, l2 = merge_literal(np.array([c["out"]]), lse, np.array([c["block_out"]]), blse)
            assert np.allclose(o2[0], c["new_out"], rtol=0, atol=1e-14)
            assert abs(l2[0] - exp_l) < 1e-14


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_blockwise_equals_one_shot(P, causal):
    rng = np.random.default_rng(P * 10 + causal)
    B, S, Hq, Hkv, d = 2, 24, 4, 2, 8
    q, k, v = _rand(rng, B, S, Hq, d, s=2), _rand(rng, B, S, Hkv, d, s=2), _rand(rng, B, S, Hkv, d)
    o_ref, l_ref = attention(q, k, v, causal=causal)
    for trial in range(3):
        splits = _random_partition(rng, S, P)
        parts = _partials(q, k, v, splits, causal)
        o, l = _fold(parts, merge_stable)
        assert np.max(np.abs(o - o_ref)) < 1e-12
        assert np.max(np.abs(l - l_ref)) < 1e-12
        if not causal:   # every partial finite -> the literal rule applies
            o2, l2 = _fold(parts, merge_literal)
            assert np.max(np.abs(o2 - o_ref)) < 1e-12
            assert np.max(np.abs(l2 - l_ref)) < 1e-12


@pytest.mark.parametrize("P", [2, 3, 4])
def test_merge_order_independence_all_orders(P):
    rng = np.random.default_rng(40 + P)
    q, k, v = _rand(rng, 1, 10, 2, 4, s=2), _rand(rng, 1, 20, 2, 4, s=2), _rand(rng, 1, 20, 2, 4)
    parts = _partials(q, k, v, _random_partition(rng, 20, P))
    o0, l0 = _fold(parts, merge_stable)
    for perm in itertools.permutations(range(P)):
        o, l = _fold([parts[i] for i in perm], merge_stable)
        assert np.max(np.abs(o - o0)) < 1e-12 and np.max(np.abs(l - l0)) < 1e-12


def test_merge_order_independence_random_orders_p8():
    rng = np.random.default_rng(48)
    q, k, v = _rand(rng, 1, 8, 2, 4, s=2), _rand(rng, 1, 32, 2, 4, s=2), _rand(rng, 1, 32, 2, 4)
    parts = _partials(q, k, v, _random_partition(rng, 32, 8))
    o0, l0 = _fold(parts, merge_stable)
    for _ in range(100):
        perm = rng.permutation(8)
        o, l = _fold([parts[i] for i in perm], merge_stable)
        assert np.max(np.abs(o - o0)) < 1e-12 and np.max(np.abs(l - l0)) < 1e-12


def test_merge_associativity_identity_self_merge():
    rng = np.random.default_rng(5)
    n, d = 50, 6
    P = [(rng.standard_normal((n, d)), rng.uniform(-40, 40, n)) for _ in range(3)]
    (a, la), (b, lb), (c, lc) = P
    left = merge_stable(*merge_stable(a, la, b, lb), c, lc)
    right = merge_stable(a, la, *merge_stable(b, lb, c, lc))
    assert np.max(np.abs(left[0] - right[0])) < 1e-12 and np.max(np.abs(left[1] - right[1])) < 1e-12
    # identity on both sides
    zero, ninf = np.zeros((n, d)), np.full(n, -np.inf)
    o, l = merge_stable(zero, ninf, a, la)
    assert np.array_equal(o, a) and np.array_equal(l, la)
    o, l = merge_stable(a, la, zero, ninf)
    assert np.array_equal(o, a) and np.array_equal(l, la)
    o, l = merge_stable(zero, ninf, zero, ninf)
    assert np.all(o == 0) and np.all(np.isneginf(l))
    # self-merge: out unchanged, lse + ln 2 (sigma(0) = 1/2)
    for rule in (merge_stable, merge_literal):
        o, l = rule(a, la, a, la)
        assert np.max(np.abs(o - a)) < 1e-12 and np.max(np.abs(l - (la + math.log(2)))) < 1e-12


def test_stable_equals_literal_where_finite_and_extremes():
    rng = np.random.default_rng(9)
    n, d = 400, 4
    a, b = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    la = rng.uniform(-60, 60, n)
    lb = la + rng.choice([-100.0, -30.0, -1e-9, 0.0, 1e-9, 30.0, 100.0], n)
    o1, l1 = merge_stable(a, la, b, lb)
    o2, l2 = merge_literal(a, la, b, lb)
    assert np.all(np.isfinite(o1)) and np.all(np.isfinite(l1))
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12
    # |difference| of 800: the literal form overflows exp(); the stable one must not
    o3, l3 = merge_stable(a, la, b, la + 800.0)
    assert np.max(np.abs(o3 - b)) < 1e-14 and np.max(np.abs(l3 - (la + 800.0))) < 1e-9
    o4, l4 = merge_stable(a, la, b, la - 800.0)
    assert np.max(np.abs(o4 - a)) < 1e-14 and np.max(np.abs(l4 - la)) < 1e-9


@pytest.mark.parametrize("layout,P,S", [("contig", 4, 32), ("contig_causal", 4, 32),
                                         ("zigzag_causal", 4, 32), ("zigzag_causal", 2, 12),
                                         ("contig", 3, 30)])
@pytest.mark.parametrize("order", ["ring", "tokenring"])
def test_ring_emulation_equals_one_shot(layout, P, S, order):
    rng = np.random.default_rng(S + P)
    q, k, v = _rand(rng, 1, S, 4, 8, s=2), _rand(rng, 1, S, 2, 8, s=2), _rand(rng, 1, S, 2, 8)
    causal = layout != "contig"
    o_ref, l_ref = attention(q, k, v, causal=causal)
    o, l = ring_blockwise(q, k, v, P, layout=layout, order=order)
    assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(l - l_ref)) < 1e-12
    if not causal:
        o2, l2 = ring_blockwise(q, k, v, P, layout=layout, order=order, rule="literal")
        assert np.max(np.abs(o2 - o_ref)) < 1e-12 and np.max(np.abs(l2 - l_ref)) < 1e-12


def test_kv_sharded_decode_equals_one_shot():
    rng = np.random.default_rng(77)
    q, k, v = _rand(rng, 3, 1, 8, 8), _rand(rng, 3, 64, 1, 8), _rand(rng, 3, 64, 1, 8)
    o_ref, l_ref = attention(q, k, v)
    o, l = ring_blockwise(q, k, v, 8, layout="kv_sharded")
    assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(l - l_ref)) < 1e-12


@pytest.mark.parametrize("Sq,Sk,P", [(1, 24, 4), (6, 24, 3), (24, 24, 4), (10, 40, 8)])
@pytest.mark.parametrize("order", ["ring", "tokenring"])
def test_kv_sharded_causal_equals_one_shot(Sq, Sk, P, order):
    """Blockwise over the K/V shards with the queries at positions
    Sk-Sq .. Sk-1 equals one-shot causal attention at those positions."""
    rng = np.random.default_rng(Sq * 100 + Sk + P)
    q, k, v = _rand(rng, 2, Sq, 4, 8, s=2), _rand(rng, 2, Sk, 2, 8, s=2), _rand(rng, 2, Sk, 2, 8)
    o_ref, l_ref = attention(q, k, v, causal=True, q_pos=np.arange(Sq) + Sk - Sq)
    o, l = ring_blockwise(q, k, v, P, layout="kv_sharded_causal", order=order)
    assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(l - l_ref)) < 1e-12


def test_kv_sharded_causal_closed_form_zero_queries():
    """Q = 0: every visible key has the same score, so query i (position
    Sk-Sq+i) gets lse = ln(Sk-Sq+i+1) and the mean of V over keys 0..Sk-Sq+i."""
    rng = np.random.default_rng(5)
    Sq, Sk, P = 7, 28, 4
    q = np.zeros((1, Sq, 2, 8))
    k, v = _rand(rng, 1, Sk, 1, 8), _rand(rng, 1, Sk, 1, 8)
    o, l = ring_blockwise(q, k, v, P, layout="kv_sharded_causal")
    for i in range(Sq):
        n = Sk - Sq + i + 1
        assert abs(l[0, 0, i] - np.log(n)) < 1e-12
        assert np.max(np.abs(o[0, i, 1] - v[0, :n, 0].mean(axis=0))) < 1e-12


def test_zigzag_balance_closed_form():
    # 2P chunks of c tokens, rank r holds chunks r and 2P-1-r: every rank sees
    # c(c+1)/2 + (r c^2) + ... which sums to 2 P c^2 + c visible pairs.
    for P, c in [(2, 3), (4, 5), (8, 7), (4, 3000)]:
        S = 2 * P * c
        counts = visible_pairs_per_rank(S, P, "zigzag_causal")
        assert counts == [2 * P * c * c + c] * P
        assert sum(counts) == S * (S + 1) // 2
    rows = zigzag_chunks(16, 4)
    assert list(rows[1]) == [2, 3, 12, 13]


def test_tokenring_schedule_golden():
    with open(os.path.join(GOLDEN, "tokenring_schedule.json")) as f:
        gold = json.load(f)
    for key in ("N4", "N8"):
        g = gold[key]
        N = g["N"]
        sch = tokenring_schedule(N)
        assert sch["compute"] == g["compute"]
        assert sch["final_send"] == g["final_send"]
        # every (owner, K/V rank) pair computed exactly once
        seen = {(sch["compute"][j][i], j) for j in range(N) for i in range(N)}
        assert len(seen) == N * N
        # owner t receives K/V ranks in ascending order t, t+1, ...
        for t in range(N):
            got = [j for i in range(N) for j in range(N) if sch["compute"][j][i] == t]
            assert got == ring_kv_order(t, N, "tokenring")
