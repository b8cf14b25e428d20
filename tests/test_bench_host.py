"""Host-side accounting of bench.py, pinned to the workload definitions.

The flop counts are the visible (query, key) pairs times 4*d*Hq*B; the
closed forms for the zigzag rank share (2Pc^2 + c pairs) are checked against
a brute-force sum over the rows that rank owns.
"""

import numpy as np
import pytest

import bench
from ring_blockwise_softmax_amd.workloads import WORKLOADS


def test_mha24k_flops():
    w = WORKLOADS["mha24k"]
    assert bench.flops_of(w) == 4.0 * 128 * 32 * 4 * 6000 * 24000 == 9437184000000.0
    assert bench.flops_of(w, rank=0) == 4.0 * 128 * 32 * 6000 * 24000


@pytest.mark.parametrize("name", ["zigzag24k", "gqa1m"])
def test_zigzag_rank_share_pairs_brute_force(name):
    w = WORKLOADS[name]
    c = w.seq_q // (2 * w.P)
    for rank in (0, w.P - 1):
        rows = bench.owned_rows(w, rank)
        assert len(rows) == 2 * c and len(np.unique(rows)) == 2 * c
        brute = int(np.sum(rows.astype(np.int64) + 1))      # causal: row i sees keys 0..i
        assert bench.visible_pairs(w, rank) == brute == 2 * w.P * c * c + c
    # all ranks together own every row once
    allrows = np.concatenate([bench.owned_rows(w, r) for r in range(w.P)])
    assert np.array_equal(np.sort(allrows), np.arange(w.seq_q))
    assert bench.visible_pairs(w) == w.seq_q * (w.seq_q + 1) // 2


def test_gqa1m_rank_share_flops():
    w = WORKLOADS["gqa1m"]
    assert bench.visible_pairs(w, 0) == 68_719_542_272
    assert abs(bench.flops_of(w, 0) - 1.1259e15) / 1.1259e15 < 1e-4


def test_decode_pairs_and_rows():
    w = WORKLOADS["mqa_decode"]
    assert bench.visible_pairs(w) == w.seq_q * w.seq_k
    assert np.array_equal(bench.owned_rows(w, -1), np.arange(w.seq_q))


def test_contig_owned_rows():
    w = WORKLOADS["mha24k"]
    n = w.seq_q // w.P
    assert np.array_equal(bench.owned_rows(w, 2), np.arange(2 * n, 3 * n))


def test_prefill_chunk_pairs_brute_force():
    w = WORKLOADS["prefill_chunk"]
    qpos = (w.seq_k - w.seq_q) + np.arange(w.seq_q, dtype=np.int64)
    assert bench.visible_pairs(w) == int(np.sum(qpos + 1))
    assert np.array_equal(bench.owned_rows(w, -1), np.arange(w.seq_q))


def test_clock_summary():
    """Clock / power summary of GPU-metrics samples: the per-XCD clocks are
    averaged per sample, the median over samples is reported, and "N/A"
    entries are dropped."""
    xcd = [1719, 1634, 1691, 1620, 1669, 1631, 1686, 1660]      # MHz, as read on an MI355X
    s = bench.summarize_clock([(xcd, 1389), (["N/A"] * 8, "N/A"), ([1600] * 8, 1380), ([1700] * 8, 1395)])
    assert s["sclk_mhz"] == 1663.8                 # median of 1600, 1663.75, 1700
    assert s["sclk_mhz_range"] == [1600.0, 1700.0]
    assert s["samples"] == 3
    assert s["socket_power_w"] == 1389
    assert bench.summarize_clock([(["N/A"], "N/A")]) is None
    assert "socket_power_w" not in bench.summarize_clock([([1500], "N/A")])


def test_dtype_override_keeps_the_shape_and_prices_fp32_against_its_peak():
    w = bench.select_workload("mha24k", "f32")
    base = WORKLOADS["mha24k"]
    assert (w.dtype, w.name) == ("f32", "mha24k_f32")
    assert (w.batch, w.heads_q, w.heads_kv, w.head_dim, w.seq_q, w.seq_k, w.P, w.layout, w.seed, w.std) == \
        (base.batch, base.heads_q, base.heads_kv, base.head_dim, base.seq_q, base.seq_k, base.P, base.layout,
         base.seed, base.std)
    assert bench.flops_of(w) == bench.flops_of(base)
    assert bench.peak_tflops(w) == bench.PEAK_F32_MFMA_TFLOPS and bench.peak_tflops(base) == bench.PEAK_BF16_TFLOPS
    # the bf16 traffic record never applies to the fp32 run
    assert bench.measured_traffic(w.name) is None
    assert bench.select_workload("mha24k", "bf16") is base and bench.select_workload("tiny") is WORKLOADS["tiny"]


def test_roofline_arithmetic():
    """achieved = algorithmic flops per launch / average launch time, frac =
    achieved / peak of the input dtype; decode is priced in K/V(+Q) bytes
    against the HBM peak.  Figures worked by hand from the definitions."""
    w = WORKLOADS["mha24k"]
    tm = {"steps": 10, "prof": {"attn": (40, 80.0)}}          # 4 launches per step, 2 ms each
    roof, launches, avg_ms = bench.roofline_of(w, -1, 2, tm)
    assert launches == 4 and avg_ms == 2.0
    assert roof["flops_per_launch"] == 9437184000000.0 / 4
    assert roof["achieved"] == round(2.359296e12 / 2e-3 / 1e12, 2) == 1179.65
    assert roof["frac"] == round(1179.65 / 2516.6, 4) and roof["unit"] == "TFLOP/s"
    f32 = bench.select_workload("mha24k", "f32")
    roof32, _, _ = bench.roofline_of(f32, -1, 4, tm)
    assert roof32["peak"] == 157.3 and roof32["frac"] == round(1179.65 / 157.3, 4)
    d = WORKLOADS["mqa_decode"]                                # B16, 262144 keys, 1 K/V head, d128, bf16
    tmd = {"steps": 20, "prof": {"attn": (20, 6.4)}}          # one launch per step, 0.32 ms
    rd, _, _ = bench.roofline_of(d, -1, 2, tmd)
    kv = 2 * 16 * 262144 * 1 * 128 * 2
    qb = 16 * 1 * 32 * 128 * 2
    assert rd["bound"] == "hbm" and rd["algorithmic_bytes_per_launch"] == kv + qb
    assert rd["achieved"] == round((kv + qb) / 0.32e-3 / 1e9, 2) and rd["peak"] == 8000.0
