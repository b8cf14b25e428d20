"""Seeded random shapes through every entry point, against the fp64 oracle.

Each case draws a dtype, head size, GQA ratio (1-8, including 3), batch, and
one of: a block (no / causal / bottom-right mask, ragged sizes down to one
row or key), an emulated ring (P up to 8 including odd P, every layout and
order, fused or not, all ranks or one rank's share), or a K/V-sharded step
(plain or causal, P up to 8, Sq up to 300).  The seed fixes everything.
"""

import numpy as np
import pytest

from oracle import attention
from oracle.blockwise import contiguous_shares, ring_blockwise, zigzag_chunks
from tests.parity import compare

pytestmark = pytest.mark.gpu

N_CASES = 200


def _case(i):
    rng = np.random.default_rng(7000 + i)
    c = {
        "dtype": str(rng.choice(["bf16", "f32"])),
        "d": int(rng.choice([64, 128])),
        "Hkv": int(rng.choice([1, 2, 3])),
        "G": int(rng.choice([1, 2, 3, 4, 8])),
        "B": int(rng.choice([1, 2])),
        "kind": str(rng.choice(["block", "ring", "kvs"])),
    }
    if c["kind"] == "block":
        Sq, Sk = int(rng.integers(1, 700)), int(rng.integers(1, 900))
        mask = str(rng.choice(["none", "causal", "causal_bottom_right"]))
        if mask == "causal":
            Sk = Sq
        if mask == "causal_bottom_right" and Sq > Sk:
            Sq, Sk = Sk, Sq
        c.update(Sq=Sq, Sk=Sk, mask=mask)
    elif c["kind"] == "ring":
        P = int(rng.choice([1, 2, 3, 4, 5, 8]))
        layout = str(rng.choice(["contig", "contig_causal", "zigzag_causal"]))
        unit = 2 * P if layout == "zigzag_causal" else P
        S = unit * int(rng.integers(1, max(2, 1200 // unit)))
        c.update(P=P, layout=layout, Sq=S, Sk=S, order=str(rng.choice(["ring", "tokenring"])),
                 fuse=bool(rng.integers(0, 2)), rank=int(rng.choice([-1, -1, 0, P - 1])))
    else:
        P = int(rng.choice([1, 2, 4, 7, 8]))
        Sk = P * int(rng.integers(1, 600))
        c.update(P=P, layout=str(rng.choice(["kv_sharded", "kv_sharded_causal"])), Sk=Sk,
                 Sq=int(rng.integers(1, min(Sk, 300) + 1)), order=str(rng.choice(["ring", "tokenring"])),
                 fuse=bool(rng.integers(0, 2)))
    return c


def _rank_rows(S, P, layout, rank):
    return (zigzag_chunks(S, P) if layout == "zigzag_causal" else contiguous_shares(S, P))[rank]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    import torch
    import ring_blockwise_softmax_amd as ra
    c = _case(i)
    print(f"[random {i}] {c}", flush=True)
    B, Sq, Sk, d, Hkv = c["B"], c["Sq"], c["Sk"], c["d"], c["Hkv"]
    Hq = Hkv * c["G"]
    tdt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    g = torch.Generator().manual_seed(9000 + i)
    q = (torch.randn(B, Sq, Hq, d, generator=g) * 0.8).to(tdt)
    k = (torch.randn(B, Sk, Hkv, d, generator=g) * 0.8).to(tdt)
    v = torch.randn(B, Sk, Hkv, d, generator=g).to(tdt)
    if c["kind"] == "block":
        out, lse = ra.block_attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask=c["mask"])
        torch.cuda.synchronize()
        qpos = np.arange(Sq) + (Sk - Sq if c["mask"] == "causal_bottom_right" else 0)
        ro, rl = attention(q, k, v, causal=(c["mask"] != "none"), q_pos=qpos)
    elif c["kind"] == "ring":
        P, rank = c["P"], c["rank"]
        out, lse = ra.ring_forward(q.cuda(), k.cuda(), v.cuda(), P, layout=c["layout"], order=c["order"],
                                   rank=rank, fuse_merge=c["fuse"])
        torch.cuda.synchronize()
        ro, rl = ring_blockwise(q.double().numpy(), k.double().numpy(), v.double().numpy(), P,
                                layout=c["layout"], order=c["order"], ranks=None if rank < 0 else [rank])
        if rank >= 0:
            rows = _rank_rows(Sq, P, c["layout"], rank)
            rows_t = torch.as_tensor(rows, device="cuda")
            out, lse, ro, rl = out[:, rows_t], lse[:, :, rows_t], ro[:, rows], rl[:, :, rows]
    else:
        out, lse = ra.ring_forward(q.cuda(), k.cuda(), v.cuda(), c["P"], layout=c["layout"], order=c["order"],
                                   fuse_merge=c["fuse"])
        torch.cuda.synchronize()
        causal = c["layout"] == "kv_sharded_causal"
        ro, rl = attention(q, k, v, causal=causal, q_pos=np.arange(Sq) + (Sk - Sq if causal else 0))
    compare(f"random {i}", out, lse, ro, rl, c["dtype"])
