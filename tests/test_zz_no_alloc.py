"""ra_block_attn_fwd_noalloc against ra_block_attn_fwd, through the C ABI.

The no-allocation entry point runs the same kernels with the split-K
partials in the library's static device scratch instead of a workspace, so
its results must equal the workspace entry point's bitwise; both are also
held to the oracle tolerances.  Two calls in a row, the second smaller, show
that what the first call left in the scratch does not leak into the second.
"""

import numpy as np
import pytest

from oracle import attention
from ring_blockwise_softmax_amd.workloads import Workload, make_inputs
from tests.parity import compare

pytestmark = pytest.mark.gpu


def _inputs(B, Sq, Sk, Hq, Hkv, d, dtype, seed):
    w = Workload("noalloc", B, Hq, Hkv, d, Sq, Sk, 1, "contig", dtype, 0.5, seed)
    return make_inputs(w, device="cuda")


# (B, Sq, Sk, Hq, Hkv, d, dtype, mask): every case is short enough in query
# rows that its keys are split over work-groups, so its partials (33 KB to
# 8.3 MB) go through the scratch; the second call of each pair is smaller.
CASES = [
    [(2, 1, 40000, 32, 1, 128, "bf16", "none"), (1, 3, 9000, 8, 2, 64, "bf16", "causal_bottom_right")],
    [(1, 2, 20000, 16, 2, 128, "f32", "none"), (1, 1, 700, 8, 8, 128, "f32", "none")],
    [(1, 300, 500, 4, 2, 128, "bf16", "causal"), (1, 130, 257, 2, 2, 64, "bf16", "none")],
]


@pytest.mark.parametrize("pair", CASES)
def test_noalloc_matches_workspace_entry_point(pair):
    import torch

    import ring_blockwise_softmax_amd as ra

    for i, (B, Sq, Sk, Hq, Hkv, d, dtype, mask) in enumerate(pair):
        print(f"[noalloc] call {i}: B{B} Sq{Sq} Sk{Sk} Hq{Hq}/Hkv{Hkv} d{d} {dtype} {mask}", flush=True)
        q, k, v = _inputs(B, Sq, Sk, Hq, Hkv, d, dtype, seed=Sq * 31 + Sk)
        if i == 0:
            need = ra.block_attn_workspace_bytes(q, k)
            print(f"[noalloc] split partials: {need} bytes", flush=True)
        ref_out, ref_lse = ra.block_attn_fwd(q, k, v, mask=mask)
        out = torch.full((B, Sq, Hq, d), float("nan"), device="cuda")
        lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
        ra.block_attn_fwd_noalloc(q, k, v, out, lse, mask=mask)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), "differs from ra_block_attn_fwd"
        qpos = np.arange(Sq) + (Sk - Sq if mask == "causal_bottom_right" else 0)
        ro, rl = attention(q.cpu(), k.cpu(), v.cpu(), causal=(mask != "none"), q_pos=qpos)
        compare(f"noalloc {B},{Sq},{Sk},{Hq}/{Hkv},d{d},{dtype},{mask}", out, lse, ro, rl, dtype)


def test_noalloc_rejects_oversized_split():
    import torch

    import ring_blockwise_softmax_amd as ra

    q, k, v = _inputs(1, 4, 32768, 32, 1, 128, "bf16", seed=1)
    assert ra.block_attn_workspace_bytes(q, k) > ra._lib.NOALLOC_SCRATCH_BYTES
    out = torch.zeros((1, 4, 32, 128), device="cuda")
    lse = torch.zeros((1, 32, 4), device="cuda")
    with pytest.raises(ra.RaError, match="static scratch"):
        ra.block_attn_fwd_noalloc(q, k, v, out, lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == 0), "a rejected call touched its outputs"
