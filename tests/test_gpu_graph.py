"""The library's enqueue sequence captured in a HIP graph and replayed.

ra_ring_forward only launches kernels on the given stream (no allocation,
no memset, no host synchronisation), so a pre-marshalled call can be
captured once and replayed.  Each replay here follows eager work that
changes the inputs in place, and every replay is checked against an eager
run on the same inputs (bitwise: same kernels, same work order).
"""

import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout,Sq,Sk,Hq,Hkv,P,fuse", [
    ("zigzag_causal", 1200, 1200, 8, 2, 4, True),     # one launch per step, fused merges
    ("contig", 960, 960, 4, 4, 4, False),             # block results through the workspace
    ("kv_sharded", 1, 16384, 32, 1, 8, True),         # decode: gather-merge (partials + reduction)
    ("kv_sharded_causal", 500, 8000, 8, 2, 8, True),  # prefill chunk
])
def test_graph_replay_matches_eager(layout, Sq, Sk, Hq, Hkv, P, fuse):
    import torch
    import ring_blockwise_softmax_amd as ra
    g = torch.Generator(device="cuda").manual_seed(31)
    q = (torch.randn(2, Sq, Hq, 128, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    k = (torch.randn(2, Sk, Hkv, 128, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    v = torch.randn(2, Sk, Hkv, 128, device="cuda", generator=g).to(torch.bfloat16)
    runner = ra.RingRunner(q, k, v, P, layout=layout, fuse_merge=fuse)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        runner.run()                       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        runner.run()
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: new inputs, written in place
        q.copy_((torch.randn(q.shape, device="cuda", generator=g) * 0.5).to(torch.bfloat16))
        v.mul_(-0.5 if rep % 2 else 1.5)
        runner.out.fill_(float("nan"))
        runner.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_l = runner.out.clone(), runner.lse.clone()
        ref_o, ref_l = ra.ring_forward(q, k, v, P, layout=layout, fuse_merge=fuse)
        torch.cuda.synchronize()
        assert torch.isfinite(got_o).all() and torch.isfinite(got_l).all(), f"replay {rep}"
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), f"replay {rep} differs from eager"
