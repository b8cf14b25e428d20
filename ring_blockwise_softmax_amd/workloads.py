"""Seeded synthetic workloads (shapes and input draws only -- no attention math).

This module is the one piece shared by the HIP path's tests/bench and the CPU
oracle's tests: it only draws random tensors and describes shapes.  It holds
none of the method's arithmetic.

Recipe (the pages fix no input distribution; they name a sequence of 24,000
tokens over a 4-rank ring and 1M-token contexts, and ask for nothing else):
one ``torch.Generator`` seeded with the workload's seed draws Q, then K, then V
with ``randn`` in fp32, multiplied by ``std`` and cast to the workload dtype.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    seq_q: int
    seq_k: int
    P: int
    layout: str            # contig | contig_causal | zigzag_causal | kv_sharded | kv_sharded_causal
    dtype: str             # "f32" | "bf16"
    std: float
    seed: int
    rank: int = -1         # -1: every rank's share; r >= 0: rank r only
    order: str = "ring"    # ring | tokenring
    gen_device: str = "cpu"
    notes: str = ""

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # B1 H1 d64, S512 over P=4 blocks of 128, non-causal, fp32 N(0,1).
    "tiny": Workload("tiny", 1, 1, 1, 64, 512, 512, 4, "contig", "f32", 1.0, 1),
    # B1 H32 d128, S24000 over P=4 blocks of 6000, non-causal, bf16 N(0,1)*0.5.
    "mha24k": Workload("mha24k", 1, 32, 32, 128, 24000, 24000, 4, "contig", "bf16", 0.5, 2),
    # Causal zigzag: 8 chunks of 3000, rank r holds chunks r and 7-r.
    "zigzag24k": Workload("zigzag24k", 1, 32, 32, 128, 24000, 24000, 4, "zigzag_causal",
                          "bf16", 0.5, 3),
    # GQA 32/8, 1,048,576 tokens over P=8, zigzag 16 chunks of 65536; rank 0's
    # share (131072 query rows) against all 8 K/V blocks.
    "gqa1m": Workload("gqa1m", 1, 32, 8, 128, 1048576, 1048576, 8, "zigzag_causal",
                      "bf16", 0.5, 4, rank=0, gen_device="cuda"),
    # MQA decode: B16, 32/1 heads, one query token against 262144 keys in
    # P=8 blocks of 32768, non-causal.
    "mqa_decode": Workload("mqa_decode", 16, 32, 1, 128, 1, 262144, 8, "kv_sharded",
                           "bf16", 0.5, 5, gen_device="cuda"),
    # Chunked prefill: the last 4096 tokens of a 131072-token context attend
    # causally (bottom-right) to K/V in P=8 shards of 16384; GQA 32/8.
    "prefill_chunk": Workload("prefill_chunk", 1, 32, 8, 128, 4096, 131072, 8, "kv_sharded_causal",
                              "bf16", 0.5, 6, gen_device="cuda"),
}


def make_inputs(w: Workload, device=None, dtype=None):
    """Draw (q, k, v) for workload ``w``: BSHD tensors, d contiguous.

    Q is [B, Sq, Hq, d]; K and V are [B, Sk, Hkv, d].  The generator lives on
    ``w.gen_device`` (large workloads are drawn on the GPU); the tensors are
    then moved to ``device`` (default: the generator's device).
    """
    import torch

    gdev = w.gen_device
    if gdev == "cuda" and not torch.cuda.is_available():
        gdev = "cpu"
    g = torch.Generator(device=gdev)
    g.manual_seed(w.seed)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype or w.dtype]

    def draw(shape):
        x = torch.randn(shape, generator=g, device=gdev, dtype=torch.float32)
        if w.std != 1.0:
            x.mul_(w.std)
        return x.to(tdt)

    q = draw((w.batch, w.seq_q, w.heads_q, w.head_dim))
    k = draw((w.batch, w.seq_k, w.heads_kv, w.head_dim))
    v = draw((w.batch, w.seq_k, w.heads_kv, w.head_dim))
    dev = device or gdev
    return q.to(dev), k.to(dev), v.to(dev)


def small(name: str, **kw) -> Workload:
    """A shrunken variant of a named workload (same recipe, smaller sizes)."""
    return WORKLOADS[name].with_(**kw)
