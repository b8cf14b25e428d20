"""The library's host planner (ra_ring_plan) against the oracle's partitions.

Pins (no GPU): every visible (query, key) pair is computed exactly once over
all ranks and steps, no fully masked chunk pair is scheduled, items of one
step write disjoint query rows, each rank's merge order is the Ring Attention
(descending) or TokenRing (ascending) order, every rank's visible-pair count
matches the oracle's direct count (zigzag: 2 P c^2 + c), and the first item
of every row range is flagged as the one that initialises it.
"""

import numpy as np
import pytest

from oracle.blockwise import ring_kv_order, visible_pairs_per_rank, zigzag_chunks, contiguous_shares


def _ra():
    import ring_blockwise_softmax_amd as ra
    return ra


def _coverage(items, S):
    cnt = np.zeros((S, S), dtype=np.int64)
    for it in items:
        q = np.arange(it["q_start"], it["q_start"] + it["q_len"])
        for sg in it["segs"]:
            k = np.arange(sg["kv_start"], sg["kv_start"] + sg["kv_len"])
            vis = np.ones((len(q), len(k)), bool)
            if sg["causal"]:
                vis = k[None, :] <= q[:, None]
            assert vis.any(), "a fully masked pair was scheduled"
            cnt[np.ix_(q, k)] += vis
    return cnt


@pytest.mark.parametrize("layout", ["contig", "contig_causal", "zigzag_causal"])
@pytest.mark.parametrize("P", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("order", ["ring", "tokenring"])
def test_plan_exact_once_coverage(layout, P, order):
    ra = _ra()
    c = 3
    S = 2 * P * c
    items = ra.ring_plan(S, S, P, layout, order)
    cnt = _coverage(items, S)
    i = np.arange(S)
    want = np.ones((S, S), np.int64) if layout == "contig" else (i[None, :] <= i[:, None]).astype(np.int64)
    assert np.array_equal(cnt, want)

    rows = zigzag_chunks(S, P) if layout == "zigzag_causal" else contiguous_shares(S, P)
    pairs = visible_pairs_per_rank(S, P, layout)
    for r in range(P):
        mine = [it for it in items if it["rank"] == r]
        # rows of the items are the rank's rows
        got_rows = set()
        for it in mine:
            got_rows.update(range(it["q_start"], it["q_start"] + it["q_len"]))
        assert got_rows == set(rows[r].tolist())
        # visible-pair count
        n = 0
        for it in mine:
            q = np.arange(it["q_start"], it["q_start"] + it["q_len"])
            for sg in it["segs"]:
                k = np.arange(sg["kv_start"], sg["kv_start"] + sg["kv_len"])
                n += int((k[None, :] <= q[:, None]).sum()) if sg["causal"] else len(q) * len(k)
        assert n == pairs[r]
        # merge order: K/V ranks by step, skipping masked ones
        order_seen = []
        for t in range(P):
            ks = {sg["kv_rank"] for it in mine if it["step"] == t for sg in it["segs"]}
            assert len(ks) <= 1
            order_seen += list(ks)
        expect = [s for s in ring_kv_order(r, P, order)
                  if not (layout == "contig_causal" and s > r)]
        assert order_seen == expect


@pytest.mark.parametrize("layout", ["contig", "contig_causal", "zigzag_causal"])
@pytest.mark.parametrize("P", [2, 4, 8])
def test_plan_step_items_disjoint_and_first_flags(layout, P):
    ra = _ra()
    S = 2 * P * 4
    items = ra.ring_plan(S, S, P, layout, "ring")
    seen = np.zeros(S, bool)
    for t in range(P):
        step = [it for it in items if it["step"] == t]
        written = np.zeros(S, np.int64)
        for it in step:
            written[it["q_start"]:it["q_start"] + it["q_len"]] += 1
        assert written.max() <= 1, "two items of one step write the same rows"
        for it in step:
            rr = slice(it["q_start"], it["q_start"] + it["q_len"])
            assert it["first"] == (not seen[rr].any())
            assert seen[rr].all() or not seen[rr].any()
        for it in step:
            seen[it["q_start"]:it["q_start"] + it["q_len"]] = True
    assert seen.all()


def test_zigzag_balance_at_config_sizes():
    ra = _ra()
    for S, P in [(24000, 4), (1048576, 8)]:
        c = S // (2 * P)
        for r in range(P):
            items = ra.ring_plan(S, S, P, "zigzag_causal", "ring", rank=r)
            n = 0
            for it in items:
                for sg in it["segs"]:
                    L = sg["kv_len"]
                    n += it["q_len"] * L if not sg["causal"] else L * (L + 1) // 2
            assert n == 2 * P * c * c + c


def test_kv_sharded_plan():
    ra = _ra()
    items = ra.ring_plan(1, 262144, 8, "kv_sharded", "ring")
    assert [it["segs"][0]["kv_rank"] for it in items] == ring_kv_order(0, 8, "ring")
    assert all(it["q_len"] == 1 and it["segs"][0]["kv_len"] == 32768 for it in items)
    assert [it["first"] for it in items] == [True] + [False] * 7
    items = ra.ring_plan(1, 262144, 8, "kv_sharded", "tokenring")
    assert [it["segs"][0]["kv_rank"] for it in items] == list(range(8))


@pytest.mark.parametrize("Sq", [1, 5, 12, 24])
@pytest.mark.parametrize("P", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("order", ["ring", "tokenring"])
def test_kv_sharded_causal_plan(Sq, P, order):
    """Queries are the last Sq of Sk positions; each visible (query, key) pair
    with key position <= query position is covered exactly once, a block is
    flagged causal exactly when some of its keys lie after the first query's
    position, and block 0 (visible to every query) comes first."""
    ra = _ra()
    Sk = 24
    items = ra.ring_plan(Sq, Sk, P, "kv_sharded_causal", order)
    assert len(items) == P
    cnt = np.zeros((Sq, Sk), dtype=np.int64)
    for it in items:
        assert it["q_start"] == 0 and it["q_len"] == Sq and it["q_pos0"] == Sk - Sq
        qpos = it["q_pos0"] + np.arange(Sq)
        (sg,) = it["segs"]
        k = np.arange(sg["kv_start"], sg["kv_start"] + sg["kv_len"])
        assert sg["causal"] == bool(k[-1] > qpos[0])
        vis = k[None, :] <= qpos[:, None] if sg["causal"] else np.ones((Sq, len(k)), bool)
        assert vis.any()
        cnt[:, k] += vis
    qpos = Sk - Sq + np.arange(Sq)
    assert np.array_equal(cnt, (np.arange(Sk)[None, :] <= qpos[:, None]).astype(np.int64))
    assert [it["segs"][0]["kv_rank"] for it in items] == ring_kv_order(0, P, order)
    assert items[0]["segs"][0]["kv_start"] == 0
    assert [it["first"] for it in items] == [True] + [False] * (P - 1)


def test_q_pos0_is_q_start_for_ring_layouts():
    ra = _ra()
    for layout in ("contig", "contig_causal", "zigzag_causal"):
        assert all(it["q_pos0"] == it["q_start"] for it in ra.ring_plan(48, 48, 4, layout))
    assert all(it["q_pos0"] == 0 for it in ra.ring_plan(3, 48, 4, "kv_sharded"))


@pytest.mark.parametrize("args", [
    (100, 100, 3, "contig"),          # S % P
    (100, 100, 4, "zigzag_causal"),   # S % 2P (100 % 8)
    (64, 32, 4, "contig"),            # Sq != Sk for a ring layout
    (1, 100, 8, "kv_sharded"),        # Sk % P
    (40, 32, 4, "kv_sharded_causal"), # Sq > Sk: queries must be the last Sq tokens
    (64, 64, 0, "contig"),            # P < 1
    (64, 64, 17, "contig"),           # P > 16
])
def test_plan_rejects(args):
    ra = _ra()
    with pytest.raises(ValueError):
        ra.ring_plan(*args)


def test_plan_rejects_bad_rank():
    ra = _ra()
    with pytest.raises(ValueError):
        ra.ring_plan(64, 64, 4, "contig", rank=4)
    with pytest.raises(ValueError):
        ra.ring_plan(1, 64, 4, "kv_sharded", rank=1)
    with pytest.raises(ValueError):
        ra.ring_plan(1, 64, 4, "kv_sharded_causal", rank=1)
