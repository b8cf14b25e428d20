"""Full-size workloads, run exactly as bench.py launches them, checked on
sampled outputs that the fp64 oracle computes one by one.

Sampled rows always include block and tile edges (first/last row of every
rank's chunk, rows 127/128 of a 128-row query tile) plus seeded random rows;
every head of a sampled row is compared unless noted.
"""

import numpy as np
import pytest

from oracle import attention
from ring_blockwise_softmax_amd.workloads import WORKLOADS, make_inputs
from tests.parity import compare, to_np

pytestmark = pytest.mark.gpu


def _ra():
    import ring_blockwise_softmax_amd as ra
    return ra


def _sample_rows(S, edges, n_random, seed):
    rng = np.random.default_rng(seed)
    rows = set(e for e in edges if 0 <= e < S)
    rows.update(rng.choice(S, size=n_random, replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def _block_edges(S, nblocks):
    n = S // nblocks
    edges = []
    for b in range(nblocks):
        edges += [b * n, b * n + 1, b * n + 127, b * n + 128, (b + 1) * n - 1]
    return edges


@pytest.mark.parametrize("order", ["ring", "tokenring"])
@pytest.mark.parametrize("fuse", [True, False])
def test_tiny_config_full(order, fuse):
    ra = _ra()
    import torch
    w = WORKLOADS["tiny"]
    q, k, v = make_inputs(w, device="cuda")
    out, lse = ra.ring_forward(q, k, v, w.P, layout=w.layout, order=order, fuse_merge=fuse)
    torch.cuda.synchronize()
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu())
    compare(f"tiny {order} fuse={fuse}", out, lse, ro, rl, "f32")


_INPUTS = {}


def _cached_inputs(w):
    """The 24k inputs are drawn on the CPU (seconds); share them between the
    variants of one workload."""
    key = (w.name, w.dtype, w.std, w.heads_q)
    if key not in _INPUTS:
        _INPUTS.clear()
        print(f"[fullsize] {w.name}: generating inputs", flush=True)
        _INPUTS[key] = make_inputs(w, device="cuda")
    return _INPUTS[key]


@pytest.mark.parametrize("order,fuse", [("ring", True), ("tokenring", True), ("ring", False)])
@pytest.mark.parametrize("name", ["mha24k", "zigzag24k", "mha24k_f32"])
def test_24k_configs_sampled(name, order, fuse):
    """mha24k_f32: the headline shape with fp32 inputs (the benchmark's
    exact-path run), 32 heads."""
    ra = _ra()
    import torch
    w = WORKLOADS[name] if name in WORKLOADS else WORKLOADS["mha24k"].with_(name=name, dtype="f32")
    q, k, v = _cached_inputs(w)
    runner = ra.RingRunner(q, k, v, w.P, layout=w.layout, order=order, rank=w.rank, fuse_merge=fuse)
    out, lse = runner.run()
    torch.cuda.synchronize()
    nb = 2 * w.P if w.layout == "zigzag_causal" else w.P
    rows = _sample_rows(w.seq_q, _block_edges(w.seq_q, nb), 24, seed=w.seed)
    print(f"[fullsize] {name} {order} fuse={fuse}: oracle on {len(rows)} rows x {w.heads_q} heads", flush=True)
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu(), causal=(w.layout != "contig"), rows=rows)
    rows_t = torch.as_tensor(rows, device="cuda")
    compare(f"{name} {order} fuse={fuse} sampled", out[:, rows_t], lse[:, :, rows_t], ro, rl, w.dtype)
    # the whole output must be finite and lse within the attainable range
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("name,order", [("mha24k", "ring"), ("zigzag24k", "tokenring")])
def test_24k_rank0_share_sampled(name, order):
    """One rank's share at full size (the shape each GPU runs in a real ring):
    its launches are one or two rounds of work-groups, which the launcher runs
    with rotating wave priorities.  Sampled rows of rank 0 against the oracle,
    and the rows rank 0 does not own stay untouched."""
    ra = _ra()
    import torch
    from oracle.blockwise import contiguous_shares, zigzag_chunks
    w = WORKLOADS[name]
    q, k, v = _cached_inputs(w)
    out = torch.full((w.batch, w.seq_q, w.heads_q, w.head_dim), 5.0, device="cuda")
    lse = torch.full((w.batch, w.heads_q, w.seq_q), 5.0, device="cuda")
    ra.ring_forward(q, k, v, w.P, layout=w.layout, order=order, rank=0, out=out, lse=lse)
    torch.cuda.synchronize()
    owned = np.asarray((zigzag_chunks(w.seq_q, w.P) if w.layout == "zigzag_causal"
                        else contiguous_shares(w.seq_q, w.P))[0], dtype=np.int64)
    rng = np.random.default_rng(w.seed + 100)
    edges = [owned[0], owned[1], owned[127], owned[128], owned[-1], owned[len(owned) // 2 - 1], owned[len(owned) // 2]]
    rows = np.array(sorted(set(int(r) for r in edges) | set(rng.choice(owned, 16, replace=False).tolist())),
                    dtype=np.int64)
    print(f"[fullsize] {name} rank 0 {order}: oracle on {len(rows)} rows x {w.heads_q} heads", flush=True)
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu(), causal=(w.layout != "contig"), rows=rows)
    rows_t = torch.as_tensor(rows, device="cuda")
    compare(f"{name} rank 0 {order} sampled", out[:, rows_t], lse[:, :, rows_t], ro, rl, w.dtype)
    not_owned = torch.ones(w.seq_q, dtype=torch.bool, device="cuda")
    not_owned[torch.as_tensor(owned, device="cuda")] = False
    assert torch.all(out[:, not_owned] == 5.0) and torch.all(lse[:, :, not_owned] == 5.0)


# The medium fp32 configuration: the 24k sequence over a 4-rank ring with 4
# heads, fp32 N(0,1) inputs (the tiny configuration's distribution), so every
# block is a 6000-key loop ending in a 16-key ragged tile (6000 = 187*32 + 16)
# and the fp32 kernel's lazy rescale runs the length of the real blocks.
MEDIUM_F32 = WORKLOADS["mha24k"].with_(name="medium_f32", heads_q=4, heads_kv=4, dtype="f32", std=1.0, seed=7)


@pytest.mark.parametrize("layout,order,fuse", [
    ("contig", "ring", True),
    ("contig", "ring", False),
    ("contig", "tokenring", True),
    ("zigzag_causal", "ring", True),
    ("zigzag_causal", "tokenring", False),
])
def test_medium_f32_sampled(layout, order, fuse):
    """fp32 at H=4, S=24000, P=4 against the oracle on >= 256 sampled rows,
    including every block's first/last rows and rows 127/128 of its tiles."""
    ra = _ra()
    import torch
    w = MEDIUM_F32.with_(layout=layout)
    q, k, v = _cached_inputs(w)
    out, lse = ra.ring_forward(q, k, v, w.P, layout=layout, order=order, fuse_merge=fuse)
    torch.cuda.synchronize()
    nb = 2 * w.P if layout == "zigzag_causal" else w.P
    rows = _sample_rows(w.seq_q, _block_edges(w.seq_q, nb), 256, seed=w.seed)
    assert len(rows) >= 256
    print(f"[fullsize] medium f32 {layout} {order} fuse={fuse}: oracle on {len(rows)} rows", flush=True)
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu(), causal=(layout != "contig"), rows=rows)
    rows_t = torch.as_tensor(rows, device="cuda")
    compare(f"medium f32 {layout} {order} fuse={fuse}", out[:, rows_t], lse[:, :, rows_t], ro, rl, "f32")
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("rank,kv_heads", [(0, (0, 7)), (7, (0, 2, 5, 7))])
def test_gqa_1m_rank_share_sampled(rank, kv_heads):
    """GQA 32/8, 1,048,576 tokens over P=8, zigzag; one rank's share only.
    Rank 0 owns chunks 0 and 15, rank 7 chunks 7 and 8 (the middle of the
    sequence, the other end of every owner's merge schedule)."""
    ra = _ra()
    import torch
    w = WORKLOADS["gqa1m"]
    print(f"[fullsize] gqa1m rank {rank}: generating inputs on the GPU", flush=True)
    q, k, v = make_inputs(w, device="cuda")
    S, P = w.seq_q, w.P
    c = S // (2 * P)
    lo, hi = rank * c, (2 * P - 1 - rank) * c   # first rows of the two owned chunks
    out = torch.full((1, S, w.heads_q, w.head_dim), float("nan"), device="cuda")
    lse = torch.full((1, w.heads_q, S), float("nan"), device="cuda")
    runner = ra.RingRunner(q, k, v, P, layout=w.layout, order=w.order, rank=rank, fuse_merge=True,
                           out=out, lse=lse)
    print(f"[fullsize] gqa1m: running rank {rank}'s share", flush=True)
    runner.run()
    torch.cuda.synchronize()
    print("[fullsize] gqa1m: done on GPU, checking", flush=True)
    # the rank's two chunks must all be written (finite), others untouched
    own = torch.cat([out[:, lo:lo + c], out[:, hi:hi + c]], dim=1)
    assert torch.isfinite(own).all()
    other = (rank + 1) * c if rank + 1 < 2 * P - 1 - rank else 0
    assert torch.isnan(out[:, other:other + 1000]).all(), "rows of other ranks were written"
    edges = [lo, lo + 1, lo + 127, lo + 128, lo + c - 1, hi, hi + 1, hi + c - 129, hi + c - 1]
    rng = np.random.default_rng(4 + rank)
    rows = sorted(set(edges) | set((lo + rng.integers(0, c, 3)).tolist()) |
                  set((hi + rng.integers(0, c, 3)).tolist()))
    rows = np.array(rows, dtype=np.int64)
    rows_t = torch.as_tensor(rows, device="cuda")
    group = w.heads_q // w.heads_kv
    for g in kv_heads:                       # each K/V head -> 4 query heads
        hs = slice(g * group, (g + 1) * group)
        print(f"[fullsize] gqa1m rank {rank}: oracle for kv head {g}, {len(rows)} rows", flush=True)
        qs = q[:, rows_t][:, :, hs].cpu()
        kk = k[:, :, g:g + 1].cpu()
        vv = v[:, :, g:g + 1].cpu()
        ro, rl = attention(qs, kk, vv, causal=True, q_pos=rows)
        compare(f"gqa1m rank{rank} kv{g}", out[:, rows_t][:, :, hs], lse[:, hs][:, :, rows_t], ro, rl, w.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_chunk_sampled(dtype):
    """Chunked prefill at full size: the last 4096 of 131072 tokens, GQA 32/8,
    K/V in 8 shards (gather-merge path), sampled rows against the oracle; also
    with fp32 inputs through the exact path."""
    ra = _ra()
    import torch
    w = WORKLOADS["prefill_chunk"]
    if dtype != w.dtype:
        w = w.with_(dtype=dtype, name=f"prefill_chunk_{dtype}")
    print("[fullsize] prefill_chunk: generating inputs on the GPU", flush=True)
    q, k, v = make_inputs(w, device="cuda")
    runner = ra.RingRunner(q, k, v, w.P, layout=w.layout, order=w.order, fuse_merge=True)
    out, lse = runner.run()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    Sq, Sk = w.seq_q, w.seq_k
    rng = np.random.default_rng(6)
    rows = np.array(sorted({0, 1, 127, 128, Sq // 2, Sq - 2, Sq - 1} | set(rng.integers(0, Sq, 3).tolist())),
                    dtype=np.int64)
    rows_t = torch.as_tensor(rows, device="cuda")
    group = w.heads_q // w.heads_kv
    for g in (0, w.heads_kv - 1):
        hs = slice(g * group, (g + 1) * group)
        print(f"[fullsize] prefill_chunk: oracle for kv head {g}, {len(rows)} rows", flush=True)
        qs = q[:, rows_t][:, :, hs].cpu()
        ro, rl = attention(qs, k[:, :, g:g + 1].cpu(), v[:, :, g:g + 1].cpu(), causal=True,
                           q_pos=rows + (Sk - Sq))
        compare(f"prefill_chunk kv{g}", out[:, rows_t][:, :, hs], lse[:, hs][:, :, rows_t], ro, rl, w.dtype)


@pytest.mark.parametrize("order,fuse,dtype", [("ring", True, "bf16"), ("tokenring", False, "bf16"),
                                              ("ring", True, "f32"), ("tokenring", False, "f32")])
def test_mqa_decode_full(order, fuse, dtype):
    """MQA decode: B16, 32/1 heads, one query vs 262144 keys over P=8 (all rows);
    also with fp32 inputs (the exact path's split-K over 32768-key blocks)."""
    ra = _ra()
    import torch
    w = WORKLOADS["mqa_decode"]
    if dtype != w.dtype:
        w = w.with_(dtype=dtype, name=f"mqa_decode_{dtype}")
    q, k, v = make_inputs(w, device="cuda")
    out, lse = ra.ring_forward(q, k, v, w.P, layout=w.layout, order=order, fuse_merge=fuse)
    torch.cuda.synchronize()
    print("[fullsize] mqa_decode: oracle over all 16 x 32 rows", flush=True)
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu())
    compare(f"mqa_decode {order} fuse={fuse}", out, lse, ro, rl, w.dtype)
