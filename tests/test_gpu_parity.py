"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Sizes are chosen so the oracle finishes in seconds while the kernels still
cross several query tiles (128 rows) and key tiles (64 / 32 keys) with a
ragged tail.  Full-size workloads are in test_gpu_fullsize.py.
"""

import numpy as np
import pytest

from oracle import attention, merge_bshd, ring_blockwise
from ring_blockwise_softmax_amd.workloads import Workload, make_inputs
from tests.parity import compare, to_np

pytestmark = pytest.mark.gpu


def _ra():
    import ring_blockwise_softmax_amd as ra
    return ra


def _inputs(B, Sq, Sk, Hq, Hkv, d, dtype, seed, std=0.5):
    w = Workload("adhoc", B, Hq, Hkv, d, Sq, Sk, 1, "contig", dtype, std, seed)
    return make_inputs(w, device="cuda")


# ---------------------------------------------------------------------------
# ra_block_attn_fwd
# ---------------------------------------------------------------------------
BLOCK_CASES = [
    # B, Sq, Sk, Hq, Hkv, d
    (1, 200, 333, 4, 2, 64),
    (2, 130, 257, 4, 4, 128),
    (1, 1, 700, 8, 1, 128),      # decode-style, packed heads
    (1, 64, 64, 2, 2, 128),
    (1, 300, 300, 8, 2, 128),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mask", ["none", "causal", "causal_bottom_right"])
@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,d", BLOCK_CASES)
def test_block_attn_matches_oracle(B, Sq, Sk, Hq, Hkv, d, mask, dtype):
    ra = _ra()
    q, k, v = _inputs(B, Sq, Sk, Hq, Hkv, d, dtype, seed=Sq * 7 + Sk, std=1.0)
    out, lse = ra.block_attn_fwd(q, k, v, mask=mask)
    import torch
    torch.cuda.synchronize()
    qpos = np.arange(Sq) + (Sk - Sq if mask == "causal_bottom_right" else 0)
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu(), causal=(mask != "none"), q_pos=qpos)
    compare(f"block {B},{Sq},{Sk},{Hq}/{Hkv},d{d},{mask}", out, lse, ro, rl, dtype)


def test_block_attn_empty_keys_and_queries():
    ra = _ra()
    import torch
    q, k, v = _inputs(1, 40, 0, 2, 2, 64, "bf16", seed=1)
    out, lse = ra.block_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    q, k, v = _inputs(1, 0, 50, 2, 2, 64, "bf16", seed=2)
    out, lse = ra.block_attn_fwd(q, k, v)
    torch.cuda.synchronize()
    assert out.numel() == 0


def test_block_attn_bottom_right_needs_sq_le_sk():
    # Bottom-right alignment with Sq > Sk is rejected; top-left causal with
    # Sq > Sk gives every row at least key 0.  Rows with no visible key only
    # arise with positions, exercised through the ring below.
    ra = _ra()
    q, k, v = _inputs(1, 10, 20, 1, 1, 64, "f32", seed=3)
    with pytest.raises(ra.RaError):
        ra.block_attn_fwd(q[:, :10], k[:, :5], v[:, :5], mask="causal_bottom_right")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_attn_adversarial_logits(dtype):
    """Sharp softmax (Q x 8), growing logits across tiles, late spikes."""
    ra = _ra()
    import torch
    B, S, H, d = 1, 300, 2, 128
    q, k, v = _inputs(B, S, S, H, H, d, dtype, seed=11, std=1.0)
    q = (q.float() * 8).to(q.dtype)
    # logits that grow with the key index: later tiles keep raising the max
    ramp = torch.linspace(0, 6, S, device="cuda")[None, :, None, None]
    k = (k.float() + ramp * q.float().mean(dim=1, keepdim=True).sign()).to(k.dtype)
    # a spike on the last key of the block
    k[:, -1] = (q.float().mean(dim=1) * 3).to(k.dtype)
    for mask in ("none", "causal"):
        out, lse = ra.block_attn_fwd(q, k, v, mask=mask)
        torch.cuda.synchronize()
        ro, rl = attention(q.cpu(), k.cpu(), v.cpu(), causal=(mask == "causal"))
        compare(f"adversarial {dtype} {mask}", out, lse, ro, rl, dtype, guard=(dtype == "bf16"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_attn_running_max_paths(dtype):
    """Rows whose maximum keeps rising by ~5 log2 units per 32-key tile (every
    tile's probabilities overflow the running reference), rising slowly,
    falling by hundreds of units (later probabilities underflow to zero), or
    flat, mixed within every wave.  The scores are exact multiples of one key
    coordinate, so only the softmax bookkeeping is under test."""
    ra = _ra()
    import torch
    B, S, H, d = 1, 2000, 2, 128
    g = torch.Generator().manual_seed(12)
    j = torch.arange(S, dtype=torch.float32)
    k = torch.randn(B, S, H, d, generator=g) * 0.5
    k[..., 0] = (1.226 * j)[None, :, None]                # s * log2(e) = 0.156 per key for q0 = 1
    q = torch.zeros(B, S, H, d)
    q[..., 0] = torch.tensor([1.0, -1.0, 0.1, 0.0])[torch.arange(S) % 4][None, :, None]
    v = torch.randn(B, S, H, d, generator=g)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = q.to(tdt).cuda(), k.to(tdt).cuda(), v.to(tdt).cuda()
    for mask in ("none", "causal"):
        out, lse = ra.block_attn_fwd(q, k, v, mask=mask)
        torch.cuda.synchronize()
        ro, rl = attention(q.cpu(), k.cpu(), v.cpu(), causal=(mask == "causal"))
        # logits reach ~300 (log2 units): fp32 rounding of the scores alone
        # exceeds the fp32 relative guard there, so fp32 keeps the contract
        compare(f"running max {dtype} {mask}", out, lse, ro, rl, dtype, guard=(dtype == "bf16"))


def test_block_attn_is_deterministic():
    ra = _ra()
    import torch
    q, k, v = _inputs(1, 513, 777, 4, 2, 128, "bf16", seed=5)
    o1, l1 = ra.block_attn_fwd(q, k, v, mask="causal")
    o2, l2 = ra.block_attn_fwd(q, k, v, mask="causal")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------------------
# ra_merge
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_merge_matches_oracle_including_infinities(d):
    ra = _ra()
    import torch
    g = torch.Generator(device="cpu").manual_seed(21)
    B, S, H = 2, 333, 4
    out = torch.randn(B, S, H, d, generator=g)
    bout = torch.randn(B, S, H, d, generator=g)
    lse = torch.randn(B, H, S, generator=g) * 30
    blse = lse + torch.tensor([-100.0, -3.0, 0.0, 1e-6, 5.0, 100.0])[torch.randint(0, 6, (B, H, S), generator=g)]
    lse[:, 0, :7] = -float("inf")          # running pair empty
    blse[:, 1, :5] = -float("inf")         # empty block
    lse[:, 2, :3] = -float("inf")
    blse[:, 2, :3] = -float("inf")         # both empty
    ro, rl = merge_bshd(out.double().numpy(), lse.double().numpy(), bout.double().numpy(),
                        blse.double().numpy())
    do, dl, dbo, dbl = out.cuda(), lse.cuda(), bout.cuda(), blse.cuda()
    ra.merge(do, dl, dbo, dbl)
    torch.cuda.synchronize()
    eo = float(np.max(np.abs(to_np(do) - ro)))
    fin = np.isfinite(rl)
    el = float(np.max(np.abs(to_np(dl)[fin] - rl[fin])))
    assert np.all(np.isneginf(to_np(dl)[~fin]))
    print(f"[parity] merge d{d}: err_out={eo:.3e} err_lse={el:.3e}")
    assert eo <= 1e-5 and el <= 1e-4


def test_merge_noncontiguous_views():
    """Strided views (a head slice) merge only their own elements."""
    ra = _ra()
    import torch
    g = torch.Generator(device="cpu").manual_seed(22)
    B, S, H, d = 1, 100, 4, 64
    out = torch.randn(B, S, H, d, generator=g).cuda()
    lse = torch.randn(B, H, S, generator=g).cuda()
    bout = torch.randn(B, S, H, d, generator=g).cuda()
    blse = torch.randn(B, H, S, generator=g).cuda()
    ref_o, ref_l = merge_bshd(to_np(out), to_np(lse), to_np(bout), to_np(blse))
    keep_o, keep_l = out.clone(), lse.clone()
    ra.merge(out[:, :, 1:3], lse[:, 1:3], bout[:, :, 1:3], blse[:, 1:3])
    torch.cuda.synchronize()
    assert np.max(np.abs(to_np(out[:, :, 1:3]) - ref_o[:, :, 1:3])) < 1e-5
    assert np.max(np.abs(to_np(lse[:, 1:3]) - ref_l[:, 1:3])) < 1e-5
    assert torch.equal(out[:, :, 0], keep_o[:, :, 0]) and torch.equal(lse[:, 3], keep_l[:, 3])


# ---------------------------------------------------------------------------
# ra_ring_forward
# ---------------------------------------------------------------------------
RING_CASES = [
    # name, B, S, Hq, Hkv, d, P, layout, dtype
    ("tiny-f32", 1, 512, 1, 1, 64, 4, "contig", "f32"),
    ("contig-bf16-ragged", 1, 1000, 4, 4, 128, 4, "contig", "bf16"),
    ("contig-f32-ragged", 1, 1000, 2, 2, 128, 4, "contig", "f32"),
    ("contig-causal-bf16", 1, 600, 4, 2, 128, 3, "contig_causal", "bf16"),
    ("zigzag-bf16", 1, 2400, 4, 4, 128, 4, "zigzag_causal", "bf16"),
    ("zigzag-gqa-bf16", 2, 960, 8, 2, 128, 4, "zigzag_causal", "bf16"),
    ("zigzag-f32-d64", 1, 768, 2, 1, 64, 4, "zigzag_causal", "f32"),
    ("zigzag-p5-bf16", 1, 2000, 2, 2, 64, 5, "zigzag_causal", "bf16"),
]


@pytest.mark.parametrize("fuse", [True, False])
@pytest.mark.parametrize("order", ["ring", "tokenring"])
@pytest.mark.parametrize("name,B,S,Hq,Hkv,d,P,layout,dtype", RING_CASES)
def test_ring_forward_matches_oracle(name, B, S, Hq, Hkv, d, P, layout, dtype, order, fuse):
    ra = _ra()
    import torch
    std = 1.0 if dtype == "f32" else 0.5
    q, k, v = _inputs(B, S, S, Hq, Hkv, d, dtype, seed=S + P, std=std)
    out, lse = ra.ring_forward(q, k, v, P, layout=layout, order=order, fuse_merge=fuse)
    torch.cuda.synchronize()
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu(), causal=(layout != "contig"))
    compare(f"ring {name} {order} fuse={fuse}", out, lse, ro, rl, dtype)


@pytest.mark.parametrize("fuse", [True, False])
@pytest.mark.parametrize("order", ["ring", "tokenring"])
@pytest.mark.parametrize("layout,S", [("zigzag_causal", 32 * 45), ("contig", 16 * 70), ("contig_causal", 16 * 50)])
def test_ring_forward_largest_ring(layout, S, order, fuse):
    """P = 16, the largest ring: the zigzag steps put 2 items per rank, 32 in
    one launch (the size of a launch's item table), with ragged tiles."""
    ra = _ra()
    import torch
    q, k, v = _inputs(1, S, S, 4, 2, 64, "bf16", seed=S + 16)
    out, lse = ra.ring_forward(q, k, v, 16, layout=layout, order=order, fuse_merge=fuse)
    torch.cuda.synchronize()
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu(), causal=(layout != "contig"))
    compare(f"ring P=16 {layout} {order} fuse={fuse}", out, lse, ro, rl, "bf16")


@pytest.mark.parametrize("fuse", [True, False])
@pytest.mark.parametrize("order", ["ring", "tokenring"])
def test_kv_sharded_without_keys(order, fuse):
    """Sk = 0 over P = 4 empty shards: every row sees no key, so it keeps the
    merge rule's identity (out = 0, lse = -inf), also after the reduction."""
    ra = _ra()
    import torch
    q, k, v = _inputs(2, 3, 0, 8, 2, 128, "bf16", seed=9)
    out = torch.full((2, 3, 8, 128), 7.0, device="cuda")
    lse = torch.full((2, 8, 3), 7.0, device="cuda")
    ra.ring_forward(q, k, v, 4, layout="kv_sharded", order=order, fuse_merge=fuse, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_empty_batch_is_a_noop():
    """B = 0: every entry point returns with nothing to do."""
    ra = _ra()
    import torch
    q, k, v = _inputs(0, 64, 64, 2, 2, 64, "bf16", seed=5)
    out, lse = ra.block_attn_fwd(q, k, v)
    assert out.shape == (0, 64, 2, 64) and lse.shape == (0, 2, 64)
    out, lse = ra.ring_forward(q, k, v, 4, layout="zigzag_causal")
    ra.merge(out, lse, out.clone(), lse.clone())
    torch.cuda.synchronize()
    assert out.numel() == 0


@pytest.mark.parametrize("rank", [0, 3])
@pytest.mark.parametrize("fuse", [True, False])
def test_ring_forward_single_rank_share(rank, fuse):
    ra = _ra()
    import torch
    from oracle.blockwise import zigzag_chunks
    S, P = 1200, 4
    q, k, v = _inputs(1, S, S, 4, 2, 128, "bf16", seed=99)
    out = torch.full((1, S, 4, 128), 7.0, device="cuda")
    lse = torch.full((1, 4, S), 7.0, device="cuda")
    ra.ring_forward(q, k, v, P, layout="zigzag_causal", rank=rank, fuse_merge=fuse, out=out, lse=lse)
    torch.cuda.synchronize()
    rows = zigzag_chunks(S, P)[rank]
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu(), causal=True, rows=rows)
    compare(f"zigzag rank {rank} fuse={fuse}", out[:, rows], lse[:, :, rows], ro, rl, "bf16")
    others = np.setdiff1d(np.arange(S), rows)
    assert torch.all(out[:, others] == 7.0) and torch.all(lse[:, :, others] == 7.0)


def test_ring_orders_agree_and_rerun_bitwise():
    ra = _ra()
    import torch
    q, k, v = _inputs(1, 1200, 1200, 4, 4, 128, "bf16", seed=7)
    o1, l1 = ra.ring_forward(q, k, v, 4, layout="zigzag_causal", order="ring")
    o2, l2 = ra.ring_forward(q, k, v, 4, layout="zigzag_causal", order="tokenring")
    o3, l3 = ra.ring_forward(q, k, v, 4, layout="zigzag_causal", order="ring")
    torch.cuda.synchronize()
    assert float((o1 - o2).abs().max()) <= 1e-5
    assert float((l1 - l2).abs().max()) <= 1e-5
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


@pytest.mark.parametrize("fuse", [True, False])
def test_kv_sharded_decode(fuse):
    """MQA decode shape, small: B=4, 32/1 heads, 1 query vs 16384 keys, P=8."""
    ra = _ra()
    import torch
    q, k, v = _inputs(4, 1, 16384, 32, 1, 128, "bf16", seed=55)
    out, lse = ra.ring_forward(q, k, v, 8, layout="kv_sharded", fuse_merge=fuse)
    torch.cuda.synchronize()
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu())
    compare(f"decode fuse={fuse}", out, lse, ro, rl, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("order", ["ring", "tokenring"])
def test_kv_sharded_gather_ragged(dtype, order):
    """Fused KV-sharded step with every block's partials gathered in one launch:
    3 queries, GQA 8/2 (heads packed into tile rows), 7 blocks of 1000 keys
    (sub-blocks end mid-tile), against one-shot attention."""
    ra = _ra()
    import torch
    q, k, v = _inputs(2, 3, 7000, 8, 2, 128, dtype, seed=57)
    out, lse = ra.ring_forward(q, k, v, 7, layout="kv_sharded", order=order, fuse_merge=True)
    torch.cuda.synchronize()
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu())
    compare(f"gather ragged {dtype} {order}", out, lse, ro, rl, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kv_sharded_gather_matches_stepwise(dtype):
    """The gather-merge (fused) and the step-by-step merge through block_out
    (unfused) agree on the decode shape.  The two cut the keys differently,
    so in bf16 each probability is rounded against a different running max:
    each path's out is within 2^-9 * max|v| of the unrounded weighted mean
    (|P~ - P| <= 2^-9 P and sum P / l = 1), so they differ by at most twice
    that.  In fp32 nothing is rounded to a narrower type and the two agree to
    fp32 accumulation order."""
    ra = _ra()
    import torch
    q, k, v = _inputs(4, 1, 16384, 32, 1, 128, dtype, seed=58)
    o1, l1 = ra.ring_forward(q, k, v, 8, layout="kv_sharded", fuse_merge=True)
    o2, l2 = ra.ring_forward(q, k, v, 8, layout="kv_sharded", fuse_merge=False)
    torch.cuda.synchronize()
    tol = 1e-5 if dtype == "f32" else 2 * 2.0 ** -9 * v.float().abs().max().item()
    assert (o1 - o2).abs().max().item() <= tol
    assert (l1 - l2).abs().max().item() <= 1e-5


KVC_CASES = [
    # B, Sq, Sk, Hq, Hkv, d, P, dtype
    (2, 1, 4096, 32, 8, 128, 8, "bf16"),      # decode step: heads packed, sub-blocks gathered
    (1, 16, 8192, 32, 8, 128, 8, "bf16"),     # 16 draft tokens: causal inside the last block
    (1, 1000, 8000, 8, 2, 128, 8, "bf16"),    # prefill chunk: 1000-key blocks end mid-tile
    (1, 300, 1200, 4, 4, 64, 4, "f32"),       # fp32 exact path, d = 64
    (1, 1200, 4800, 4, 4, 64, 4, "bf16"),     # d = 64, 4800 rows x 16 partials: row-parallel reduction
]


@pytest.mark.parametrize("fuse", [True, False])
@pytest.mark.parametrize("order", ["ring", "tokenring"])
@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,d,P,dtype", KVC_CASES)
def test_kv_sharded_causal_matches_oracle(B, Sq, Sk, Hq, Hkv, d, P, dtype, order, fuse):
    """Queries at the last Sq of Sk positions against K/V cut into P shards,
    causal on positions, against one-shot causal attention at those positions."""
    ra = _ra()
    import torch
    q, k, v = _inputs(B, Sq, Sk, Hq, Hkv, d, dtype, seed=60 + Sq)
    out, lse = ra.ring_forward(q, k, v, P, layout="kv_sharded_causal", order=order, fuse_merge=fuse)
    torch.cuda.synchronize()
    ro, rl = attention(q.cpu(), k.cpu(), v.cpu(), causal=True, q_pos=np.arange(Sq) + Sk - Sq)
    compare(f"kv_sharded_causal B{B} Sq{Sq} Sk{Sk} {dtype} {order} fuse={fuse}", out, lse, ro, rl, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fuse", [True, False])
def test_kv_sharded_causal_closed_form(dtype, fuse):
    """Q = 0 makes every visible key score 0, and V's first coordinate holds
    the key position / 64: query i (position Sk-Sq+i) must get lse = ln(n) and
    out[..., 0] = (n-1)/128 with n = Sk-Sq+i+1 visible keys -- an off-by-one
    in the bottom-right mask moves lse by ~1/n and out by 1/128."""
    ra = _ra()
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, Sq, Sk, Hq, Hkv, d, P = 1, 40, 64, 4, 2, 64, 4
    g = torch.Generator().manual_seed(61)
    q = torch.zeros(B, Sq, Hq, d)
    k = torch.randn(B, Sk, Hkv, d, generator=g)
    v = torch.randn(B, Sk, Hkv, d, generator=g)
    v[..., 0] = (torch.arange(Sk, dtype=torch.float32) / 64.0)[None, :, None]
    q, k, v = q.to(tdt).cuda(), k.to(tdt).cuda(), v.to(tdt).cuda()
    out, lse = ra.ring_forward(q, k, v, P, layout="kv_sharded_causal", fuse_merge=fuse)
    torch.cuda.synchronize()
    n = (Sk - Sq + np.arange(Sq) + 1).astype(np.float64)
    got_lse = lse.double().cpu().numpy()            # [B, Hq, Sq]
    got0 = out[..., 0].double().cpu().numpy()      # [B, Sq, Hq]
    assert np.max(np.abs(got_lse - np.log(n)[None, None, :])) <= 1e-5
    # bf16 rounds P = 1 exactly, so both paths reproduce the mean to fp32 rounding
    assert np.max(np.abs(got0 - ((n - 1) / 128.0)[None, :, None])) <= 1e-5


def test_oracle_ring_emulation_matches_gpu_ring():
    """The oracle's own ring emulation (blockwise) and the GPU agree too."""
    ra = _ra()
    import torch
    q, k, v = _inputs(1, 480, 480, 2, 2, 64, "f32", seed=8, std=1.0)
    out, lse = ra.ring_forward(q, k, v, 4, layout="zigzag_causal", order="tokenring")
    torch.cuda.synchronize()
    ro, rl = ring_blockwise(to_np(q), to_np(k), to_np(v), 4, layout="zigzag_causal", order="tokenring")
    compare("ring emulation oracle vs gpu", out, lse, ro, rl, "f32")


def test_side_stream_call_keeps_its_workspace():
    """A call on a stream other than torch's current one: outputs and the
    temporary split-K workspace are allocated on the current stream, so the
    binding marks them used by the call's stream; memory allocated on the
    current stream right after the call must not overwrite them while the
    side stream's kernels still run."""
    ra = _ra()
    import torch
    q, k, v = _inputs(4, 1, 60000, 32, 1, 128, "bf16", seed=31)
    assert ra.block_attn_workspace_bytes(q, k) > 0
    ref_o, ref_l = ra.block_attn_fwd(q, k, v)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, l = ra.block_attn_fwd(q, k, v, stream=side)
    junk = [torch.full((1 << 20,), float("nan"), device="cuda") for _ in range(16)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_concurrent_host_threads_on_two_streams():
    """Two host threads call the library at the same time on two streams of
    default priority (first-use kernel set-up, the device-attribute cache and
    the launch path run concurrently); each result is bitwise equal to the same
    call made alone on the current stream."""
    import threading
    import torch
    ra = _ra()
    cases = [(2400, "zigzag_causal", "bf16", 11), (1000, "contig", "f32", 12)]
    inputs = [_inputs(1, S, S, 4, 2, 128, dt, seed=sd) for S, _, dt, sd in cases]
    ref = [ra.ring_forward(q, k, v, 4, layout=lay) for (q, k, v), (_, lay, _, _) in zip(inputs, cases)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [None, None]
    barrier = threading.Barrier(2)

    def worker(i):
        q, k, v = inputs[i]
        barrier.wait()
        with torch.cuda.stream(streams[i]):
            res = []
            for _ in range(5):
                res.append(ra.ring_forward(q, k, v, 4, layout=cases[i][1], stream=streams[i]))
            got[i] = res

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for i in range(2):
        for out, lse in got[i]:
            assert torch.equal(out, ref[i][0]) and torch.equal(lse, ref[i][1]), f"case {i}"
