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


@pytest.mark.parametrize("name", ["mha24k", "zigzag24k"])
def test_24k_configs_sampled(name):
    ra = _ra()
    import torch
    w = WORKLOADS[name]
    print(f"[fullsize] {name}: generating inputs", flush=True)
    q, k, v = make_inputs(w, device="cuda")
    runner = ra.RingRunner(q, k, v, w.P, layout=w.layout, order=w.order, rank=w.rank, fuse_merge=True)
    out, lse = runner.run()
    torch.cuda.synchronize()
    nb = 2 * w.P if w.layout == "zigzag_causal" else w.P
    rows = _sample_rows(w.seq_q, _block_edges(w.seq_q, nb), 24, seed=w.seed)
    print(f"[fullsize] {name}: oracle on {len(rows)} rows x {w.heads_q} heads", flush=True)
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu(), causal=(w.layout != "contig"), rows=rows)
    rows_t = torch.as_tensor(rows, device="cuda")
    compare(f"{name} sampled", out[:, rows_t], lse[:, :, rows_t], ro, rl, w.dtype)
    # the whole output must be finite and lse within the attainable range
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()


def test_gqa_1m_rank0_share_sampled():
    """GQA 32/8, 1,048,576 tokens over P=8, zigzag; rank 0's share only."""
    ra = _ra()
    import torch
    w = WORKLOADS["gqa1m"]
    print("[fullsize] gqa1m: generating inputs on the GPU", flush=True)
    q, k, v = make_inputs(w, device="cuda")
    S, P = w.seq_q, w.P
    c = S // (2 * P)
    out = torch.full((1, S, w.heads_q, w.head_dim), float("nan"), device="cuda")
    lse = torch.full((1, w.heads_q, S), float("nan"), device="cuda")
    runner = ra.RingRunner(q, k, v, P, layout=w.layout, order=w.order, rank=0, fuse_merge=True,
                           out=out, lse=lse)
    print("[fullsize] gqa1m: running rank 0's share", flush=True)
    runner.run()
    torch.cuda.synchronize()
    print("[fullsize] gqa1m: done on GPU, checking", flush=True)
    # rank 0 owns chunks 0 and 2P-1; its rows must all be written (finite)
    own = torch.cat([out[:, :c], out[:, (2 * P - 1) * c:]], dim=1)
    assert torch.isfinite(own).all()
    assert torch.isnan(out[:, c:c + 1000]).all(), "rows of other ranks were written"
    edges = [0, 1, 127, 128, c - 1, (2 * P - 1) * c, (2 * P - 1) * c + 1, S - 129, S - 1]
    rng = np.random.default_rng(4)
    rows = sorted(set(edges) | set(rng.integers(0, c, 3).tolist()) |
                  set(((2 * P - 1) * c + rng.integers(0, c, 3)).tolist()))
    rows = np.array(rows, dtype=np.int64)
    rows_t = torch.as_tensor(rows, device="cuda")
    group = w.heads_q // w.heads_kv
    for g in (0, w.heads_kv - 1):            # two K/V heads -> 8 query heads
        hs = slice(g * group, (g + 1) * group)
        print(f"[fullsize] gqa1m: oracle for kv head {g}, {len(rows)} rows", flush=True)
        qs = q[:, rows_t][:, :, hs].cpu()
        kk = k[:, :, g:g + 1].cpu()
        vv = v[:, :, g:g + 1].cpu()
        ro, rl = attention(qs, kk, vv, causal=True, q_pos=rows)
        compare(f"gqa1m rank0 kv{g}", out[:, rows_t][:, :, hs], lse[:, hs][:, :, rows_t], ro, rl, w.dtype)


def test_prefill_chunk_sampled():
    """Chunked prefill at full size: the last 4096 of 131072 tokens, GQA 32/8,
    K/V in 8 shards (gather-merge path), sampled rows against the oracle."""
    ra = _ra()
    import torch
    w = WORKLOADS["prefill_chunk"]
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


@pytest.mark.parametrize("order,fuse", [("ring", True), ("tokenring", False)])
def test_mqa_decode_full(order, fuse):
    """MQA decode: B16, 32/1 heads, one query vs 262144 keys over P=8 (all rows)."""
    ra = _ra()
    import torch
    w = WORKLOADS["mqa_decode"]
    q, k, v = make_inputs(w, device="cuda")
    out, lse = ra.ring_forward(q, k, v, w.P, layout=w.layout, order=order, fuse_merge=fuse)
    torch.cuda.synchronize()
    print("[fullsize] mqa_decode: oracle over all 16 x 32 rows", flush=True)
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu())
    compare(f"mqa_decode {order} fuse={fuse}", out, lse, ro, rl, w.dtype)
