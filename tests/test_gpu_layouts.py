"""Strided memory layouts through the C ABI, against the fp64 oracle.

The descriptors carry (batch, token, head) strides; these cases put Q, K, V,
out and lse inside larger buffers the way callers hold them: one packed QKV
projection, a K/V cache longer than the attended prefix, an output that is a
slice of a wider activation, and an lse slice of a longer row buffer.
"""

import numpy as np
import pytest

from oracle import attention
from tests.parity import compare

pytestmark = pytest.mark.gpu


def _ra():
    import ring_blockwise_softmax_amd as ra
    return ra


def _randn(shape, seed, std, dtype):
    import torch
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(dtype)


def _dense(t):
    return t.contiguous().cpu()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_packed_qkv_block_attention(dtype):
    """q, k, v are head slices of one [B, S, Hq + 2 Hkv, d] projection."""
    ra = _ra()
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, S, Hq, Hkv, d = 2, 300, 4, 2, 128
    qkv = _randn((B, S, Hq + 2 * Hkv, d), 7, 0.5, tdt).cuda()
    q, k, v = qkv[:, :, :Hq], qkv[:, :, Hq:Hq + Hkv], qkv[:, :, Hq + Hkv:]
    assert not q.is_contiguous() and q.stride(1) == (Hq + 2 * Hkv) * d
    out, lse = ra.block_attn_fwd(q, k, v, mask="causal")
    torch.cuda.synchronize()
    ro, rl = attention(_dense(q), _dense(k), _dense(v), causal=True)
    compare(f"packed qkv block {dtype}", out, lse, ro, rl, dtype)


def test_packed_qkv_zigzag_ring():
    """The emulated zigzag ring over a packed QKV projection (GQA 8/2)."""
    ra = _ra()
    import torch
    B, S, Hq, Hkv, d, P = 1, 1600, 8, 2, 128, 4
    qkv = _randn((B, S, Hq + 2 * Hkv, d), 8, 0.5, torch.bfloat16).cuda()
    q, k, v = qkv[:, :, :Hq], qkv[:, :, Hq:Hq + Hkv], qkv[:, :, Hq + Hkv:]
    for order in ("ring", "tokenring"):
        out, lse = ra.ring_forward(q, k, v, P, layout="zigzag_causal", order=order, fuse_merge=True)
        torch.cuda.synchronize()
        ro, rl = attention(_dense(q), _dense(k), _dense(v), causal=True)
        compare(f"packed qkv zigzag {order}", out, lse, ro, rl, "bf16")


def test_kv_cache_prefix_and_strided_outputs():
    """K/V are the first Sk rows of a longer cache (batch stride > Sk rows);
    out is a head slice of a wider fp32 buffer and lse a slice of longer rows."""
    ra = _ra()
    import torch
    B, Sq, Sk, Scache, Hq, Hkv, d = 3, 130, 700, 1024, 4, 1, 64
    q = _randn((B, Sq, Hq, d), 9, 0.5, torch.bfloat16).cuda()
    kc = _randn((B, Scache, Hkv, d), 10, 0.5, torch.bfloat16).cuda()
    vc = _randn((B, Scache, Hkv, d), 11, 0.5, torch.bfloat16).cuda()
    k, v = kc[:, :Sk], vc[:, :Sk]
    wide = torch.full((B, Sq, Hq + 4, d), 123.0, device="cuda")
    out = wide[:, :, 2:2 + Hq]
    lbuf = torch.full((B, Hq, Sq + 40), 123.0, device="cuda")
    lse = lbuf[:, :, 8:8 + Sq]
    ra.block_attn_fwd(q, k, v, mask="causal_bottom_right", out=out, lse=lse)
    torch.cuda.synchronize()
    qpos = np.arange(Sq) + (Sk - Sq)
    ro, rl = attention(_dense(q), _dense(k), _dense(v), causal=True, q_pos=qpos)
    compare("kv cache prefix, strided out/lse", out, lse, ro, rl, "bf16")
    # bytes outside the views are untouched
    assert torch.all(wide[:, :, :2] == 123.0) and torch.all(wide[:, :, 2 + Hq:] == 123.0)
    assert torch.all(lbuf[:, :, :8] == 123.0) and torch.all(lbuf[:, :, 8 + Sq:] == 123.0)


def test_merge_into_strided_running_state():
    """merge() folds a contiguous partial into (out, lse) held as strided views."""
    ra = _ra()
    import torch
    from oracle import merge_bshd
    B, S, H, d = 2, 257, 3, 128
    wide = _randn((B, S, H + 2, d), 12, 1.0, torch.float32).cuda()
    out = wide[:, :, 1:1 + H]
    lbuf = _randn((B, H, S + 16), 13, 2.0, torch.float32).cuda()
    lse = lbuf[:, :, 16:]
    bout = _randn((B, S, H, d), 14, 1.0, torch.float32).cuda()
    blse = _randn((B, H, S), 15, 2.0, torch.float32).cuda()
    o0, l0 = out.double().cpu().numpy(), lse.double().cpu().numpy()
    ra.merge(out, lse, bout, blse)
    torch.cuda.synchronize()
    ro, rl = merge_bshd(o0, l0, bout.double().cpu().numpy(), blse.double().cpu().numpy())
    assert np.abs(out.double().cpu().numpy() - ro).max() <= 1e-5
    assert np.abs(lse.double().cpu().numpy() - rl).max() <= 1e-5


def test_mfma_probe_library_runs():
    """The benchmark's MFMA-only probe (libra_probe.so) runs both operand
    modes: zero operands give exact zeros; random operands give finite sums."""
    import ctypes
    import os
    import torch
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib = ctypes.CDLL(os.path.join(root, "ring_blockwise_softmax_amd", "libra_probe.so"))
    g = torch.Generator(device="cuda").manual_seed(2)
    src = (torch.randn(1024 * 8, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    grid = 16
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for zero in (1, 0):
        sink = torch.full((grid * 256,), float("nan"), device="cuda")
        assert lib.ra_probe_mfma_loop(zero, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(sink.data_ptr()),
                                      grid, 4, stream) == 0
        torch.cuda.synchronize()
        assert torch.isfinite(sink).all()
        if zero:
            assert torch.all(sink == 0)
        else:
            assert float(sink.abs().max()) > 0
