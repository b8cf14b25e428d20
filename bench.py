"""Benchmark: exact ring-emulated blockwise attention on one MI355X.

Default workload (the headline): B=1, H=32, d=128, S=24000 over a P=4 ring
(4 blocks of 6000 tokens), non-causal, bf16 Q/K/V ~ N(0,1)*0.5, fp32 out/lse.
One step = one ra_ring_forward call that emulates every rank: 4 ring steps,
each one attention launch over the 4 ranks' (Q block, K/V block) pairs with
the sigma-rule merge fused into its epilogue.  Inputs are resident in HBM
before timing starts.

Prints ONE JSON line.  Extra objects:
  roofline      -- the attention kernel: algorithmic flops per launch divided
                   by its average launch time (HIP events on the launch stream
                   during the timed region), against the bf16 dense MFMA peak;
                   for the decode workload, K/V (+Q) bytes per launch against
                   the HBM peak.
  step_ms       -- min / median / max of per-step times (one event pair per
                   step, a separate region from the timed one).
  roofline.ceiling -- the kernel's matrix instruction alone on random bf16
                   operands (a probe library), its TFLOP/s, clock and power,
                   and frac_of_ceiling = achieved / that rate; the same loop
                   on zero operands runs at full clock for comparison.
  clock         -- per-XCD gfx clock (median of the XCD means) and socket
                   power from the GPU metrics while the same steps run for
                   ~2 s after the timed regions; roofline.frac_at_sclk is
                   the kernel against the MFMA peak at that clock (the
                   nominal peak assumes 2.4 GHz).
  merge         -- the standalone merge kernel at the GQA 1M-token share shape
                   (4,194,304 row-heads x d128, 6.49 GB moved), in GB/s.
  f32_path      -- (headline only) the same shape with fp32 inputs through
                   the fp32 exact path: ring time and the attention launch
                   against the 157.3 TFLOP/s fp32 MFMA peak.
  other_workloads -- (headline only) the mha24k rank-0 share, zigzag24k
                   (all ranks and the rank-0 share), gqa1m (rank-0 share),
                   mqa_decode and prefill_chunk, each as --workload NAME
                   [--rank R] runs it, in compact form: ms per step, TFLOP/s,
                   and the attention kernel against its roofline.
Profiling runs of the headline pass --no-f32 --no-others so the kernel
statistics hold the headline's launches only.
  cpu_baseline  -- the fp64 CPU oracle on a bounded sample of the same
                   workload (query rows x all keys), scaled to TFLOP/s; its
                   "check" compares the GPU result on those rows with the
                   oracle's (max abs errors, max |oracle out|).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk (AMD's "2.5 PF" dense bf16)
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

KERNEL_SRC = os.path.join(ROOT, "ring_blockwise_softmax_amd", "csrc", "ra_kernels.hip")
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attn_bf16_mha24k_traffic.json")
CALIB_BYTES = 1 << 30


def kernel_source_sha256():
    import hashlib

    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 record.

    The record holds FETCH_SIZE and WRITE_SIZE of the kernel (KiB per
    dispatch) and of a plain device copy of CALIB_BYTES, measured with the
    commands it names.  It only applies to the kernel source it was taken
    on (SHA-256 of ra_kernels.hip); otherwise the traffic is unknown (None).
    """
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha256() or rec.get("workload") != workload:
        return None
    f_fetch = rec["calib_bytes"] / (rec["calib_fetch_kib"] * 1024.0)
    f_write = rec["calib_bytes"] / (rec["calib_write_kib"] * 1024.0)
    return (rec["attn_fetch_kib"] * f_fetch + rec["attn_write_kib"] * f_write) * 1024.0


def visible_pairs(w, rank=None):
    """Visible (query, key) pairs of the emulated ranks."""
    S, P = w.seq_q, w.P
    if w.layout == "contig":
        n = S // P
        ranks = range(P) if (rank is None or rank < 0) else [rank]
        return len(list(ranks)) * n * S
    if w.layout == "kv_sharded":
        return w.seq_q * w.seq_k
    if w.layout == "kv_sharded_causal":
        # query i sits at position Sk - Sq + i and sees that many keys plus one
        return w.seq_q * (w.seq_k - w.seq_q) + w.seq_q * (w.seq_q + 1) // 2
    # causal layouts: query at position i sees i+1 keys
    if w.layout == "zigzag_causal":
        c = S // (2 * P)
        if rank is None or rank < 0:
            return S * (S + 1) // 2
        return 2 * P * c * c + c
    if w.layout == "contig_causal":
        n = S // P
        if rank is None or rank < 0:
            return S * (S + 1) // 2
        lo, hi = rank * n, (rank + 1) * n
        return sum(i + 1 for i in range(lo, hi))
    raise ValueError(w.layout)


def select_workload(name, dtype=None):
    """The named workload, optionally with its inputs in another dtype (same
    shape, seed and value recipe).  A changed dtype also changes the name, so
    a traffic record taken on the named workload is not applied to it."""
    from ring_blockwise_softmax_amd.workloads import WORKLOADS

    w = WORKLOADS[name]
    if dtype is not None and dtype != w.dtype:
        w = w.with_(dtype=dtype, name=f"{w.name}_{dtype}")
    return w


def peak_tflops(w):
    """The dense MFMA peak the attention kernel of workload w is priced against."""
    return PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS


def flops_of(w, rank=None):
    return 4.0 * w.head_dim * w.heads_q * w.batch * visible_pairs(w, rank)


def owned_rows(w, rank):
    """Query rows whose (out, lse) the emulated rank(s) produce."""
    import numpy as np

    S, P = w.seq_q, w.P
    if rank is None or rank < 0 or w.layout.startswith("kv_sharded"):
        return np.arange(S)
    if w.layout == "zigzag_causal":
        c = S // (2 * P)
        return np.concatenate([np.arange(rank * c, (rank + 1) * c),
                               np.arange((2 * P - 1 - rank) * c, (2 * P - rank) * c)])
    n = S // P
    return np.arange(rank * n, (rank + 1) * n)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, q, k, v, out=None, lse=None, rank=None, budget_s=12.0):
    """Time the oracle on a bounded sample of query rows against all keys.

    When the GPU result (out, lse) is given, the same sampled rows are also
    compared with the oracle's values (max abs errors and max |oracle out|).
    """
    import numpy as np

    from oracle import attention

    try:
        from threadpoolctl import threadpool_info

        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    kc, vc = k.cpu(), v.cpu()
    causal = w.layout != "contig" and w.layout != "kv_sharded"
    q_shift = w.seq_k - w.seq_q if w.layout == "kv_sharded_causal" else 0  # query positions
    S = w.seq_q
    pool = owned_rows(w, rank)
    rng = np.random.default_rng(0)
    rows = 16
    total_rows, total_t = 0, 0.0
    err_out = err_lse = max_ref = 0.0
    while total_t < budget_s and total_rows < len(pool):
        sel = np.sort(rng.choice(pool, size=min(rows, len(pool)), replace=False))
        qs = q[:, sel].cpu()
        t0 = time.perf_counter()
        ro, rl = attention(qs, kc, vc, causal=causal, q_pos=sel + q_shift)
        dt = time.perf_counter() - t0
        if out is not None:
            go = out[:, sel].double().cpu().numpy()
            gl = lse[:, :, sel].double().cpu().numpy()
            err_out = max(err_out, float(np.max(np.abs(go - ro))))
            err_lse = max(err_lse, float(np.max(np.abs(gl - rl))))
            max_ref = max(max_ref, float(np.max(np.abs(ro))))
        total_rows += len(sel)
        total_t += dt
        rows = min(rows * 2, 4096)
        if dt > budget_s / 2:
            break
    # flops of the sampled rows: each sees all keys (non-causal) -> scale by
    # the workload's mean keys per row otherwise
    keys_per_row = visible_pairs(w) / (w.seq_q * 1.0) if causal else w.seq_k
    fl = 4.0 * w.head_dim * w.heads_q * w.batch * total_rows * keys_per_row
    rec = {
        "value": fl / total_t / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{total_rows} query rows x {w.heads_q} heads x all {w.seq_k} keys "
                  f"(of {w.seq_q} rows), fp64 numpy, {total_t:.1f} s",
        "cpu": cpu_model(),
    }
    # one single-threaded run of the oracle on the first sampled rows
    try:
        from threadpoolctl import threadpool_limits

        sel = np.sort(rng.choice(pool, size=min(16, len(pool)), replace=False))
        qs = q[:, sel].cpu()
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            attention(qs, kc, vc, causal=causal, q_pos=sel + q_shift)
            dt1 = time.perf_counter() - t0
        rec["single_thread"] = {"value": 4.0 * w.head_dim * w.heads_q * w.batch * len(sel) * keys_per_row / dt1 / 1e12,
                                "unit": "TFLOP/s", "sample": f"{len(sel)} query rows, {dt1:.1f} s"}
    except ImportError:
        pass
    if out is not None:
        rec["check"] = {"rows": total_rows, "max_err_out": err_out, "max_abs_oracle_out": max_ref,
                        "max_err_lse": err_lse}
    return rec


def _gpu_ms(run, n=5):
    """Median time of run() over n event-timed calls after two warm-up calls."""
    import torch

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ts = []
    for _ in range(n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return sorted(ts)[len(ts) // 2]


def oracle_table():
    """The fp64 oracle timed per configuration beside the GPU (one JSON line
    each): the tiny ring, the 24k MHA rank-0 share and full ring, the 24k
    zigzag rank-0 share and the MQA decode step in full; the 1M-token GQA
    rank-0 share on 64 query rows x 32 heads (chunk edges plus random rows of
    both of rank 0's chunks), extrapolated to its 131072 rows.  Each line has
    the oracle's wall time and rate with the threads it used, a single-thread
    rate on 16 of the same rows (2 for the 1M-token share), the GPU time of the same work and the GPU
    result's error on the rows the oracle computed."""
    import numpy as np
    import torch

    import ring_blockwise_softmax_amd as ra
    from oracle import attention
    from ring_blockwise_softmax_amd.workloads import WORKLOADS, make_inputs

    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [os.cpu_count()])
    except ImportError:
        threadpool_limits, threads = None, os.cpu_count()

    def one(name, rank, parts, extrapolate_to=None, label=None, st_rows=16):
        w = WORKLOADS[name]
        print(f"[oracle-table] {label or name}: inputs", file=sys.stderr, flush=True)
        q, k, v = make_inputs(w, device="cuda")
        runner = ra.RingRunner(q, k, v, w.P, layout=w.layout, order=w.order, rank=rank, fuse_merge=True)
        gpu_ms = _gpu_ms(runner.run)
        out, lse = runner.out, runner.lse
        torch.cuda.synchronize()
        causal = w.layout not in ("contig", "kv_sharded")
        q_shift = w.seq_k - w.seq_q if w.layout == "kv_sharded_causal" else 0
        kc, vc = k.cpu(), v.cpu()
        t_total, n_rows, eo, el, mo = 0.0, 0, 0.0, 0.0, 0.0
        for i, rows in enumerate(parts):
            qs = q[:, torch.as_tensor(rows, device="cuda")].cpu()
            t0 = time.perf_counter()
            ro, rl = attention(qs, kc, vc, causal=causal, q_pos=rows + q_shift)
            dt = time.perf_counter() - t0
            t_total += dt
            n_rows += len(rows)
            rt = torch.as_tensor(rows, device="cuda")
            go = out[:, rt].double().cpu().numpy()
            gl = lse[:, :, rt].double().cpu().numpy()
            eo = max(eo, float(np.max(np.abs(go - ro))))
            el = max(el, float(np.max(np.abs(gl - rl))))
            mo = max(mo, float(np.max(np.abs(ro))))
            print(f"[oracle-table] {label or name}: part {i + 1}/{len(parts)} ({len(rows)} rows) {dt:.1f} s",
                  file=sys.stderr, flush=True)
        keys_per_row = visible_pairs(w) / (w.seq_q * 1.0) if causal else w.seq_k
        if w.layout == "zigzag_causal" and rank is not None and rank >= 0:
            keys_per_row = visible_pairs(w, rank) / (len(owned_rows(w, rank)) * 1.0)
        fl = 4.0 * w.head_dim * w.heads_q * w.batch * n_rows * keys_per_row
        rec = {"config": label or name, "rows_timed": n_rows * w.batch, "heads": w.heads_q,
               "keys": w.seq_k, "oracle_s": round(t_total, 2), "oracle_tflops": fl / t_total / 1e12,
               "cores": int(threads), "cpu": cpu_model(), "gpu_ms": round(gpu_ms, 4),
               "check": {"max_err_out": eo, "max_abs_oracle_out": mo, "max_err_lse": el}}
        if extrapolate_to:
            rec["oracle_s_extrapolated"] = round(t_total * extrapolate_to / n_rows, 1)
            rec["extrapolated_from"] = f"{n_rows} rows x {w.heads_q} heads to {extrapolate_to} rows"
        rec["speedup_gpu_vs_oracle"] = round(rec.get("oracle_s_extrapolated", t_total) / (gpu_ms / 1e3), 1)
        if threadpool_limits is not None:
            sel = parts[0][:st_rows]
            qs = q[:, torch.as_tensor(sel, device="cuda")].cpu()
            with threadpool_limits(limits=1):
                t0 = time.perf_counter()
                attention(qs, kc, vc, causal=causal, q_pos=sel + q_shift)
                dt1 = time.perf_counter() - t0
            rec["single_thread_tflops"] = 4.0 * w.head_dim * w.heads_q * w.batch * len(sel) * keys_per_row / dt1 / 1e12
        print(json.dumps(rec), flush=True)
        del q, k, v, kc, vc, runner, out, lse
        torch.cuda.empty_cache()

    one("tiny", -1, [np.arange(512)])
    one("mha24k", 0, [np.arange(6000)], label="mha24k rank-0 share")
    one("mha24k", -1, [np.arange(r * 6000, (r + 1) * 6000) for r in range(4)], label="mha24k full ring")
    one("zigzag24k", 0, [owned_rows(WORKLOADS["zigzag24k"], 0)], label="zigzag24k rank-0 share")
    w4 = WORKLOADS["gqa1m"]
    c = w4.seq_q // (2 * w4.P)
    hi = (2 * w4.P - 1) * c
    rng = np.random.default_rng(4)
    edges = [0, 1, 127, 128, c - 1, hi, hi + 1, hi + 127, hi + 128, w4.seq_q - 1]
    rest = np.concatenate([rng.choice(np.arange(2, c - 1), 27, replace=False),
                           rng.choice(np.arange(hi + 2, w4.seq_q - 1), 27, replace=False)])
    rows4 = np.unique(np.concatenate([edges, rest]))[:64]
    one("gqa1m", 0, [rows4], extrapolate_to=2 * c, label="gqa1m rank-0 share (sampled)", st_rows=2)
    one("mqa_decode", -1, [np.arange(1)], label="mqa_decode")


def traffic_probe():
    """A fixed sequence of launches for per-dispatch counter runs (rocprofv3
    --pmc): a 1 GiB device copy (counter calibration); twice a write-only
    block launch of the 24k step's shape (B4 H32, 6000 x 6000: K/V re-read by
    47 query tiles); twice the same keys against 128 query rows (K/V read by
    a single work-group); one fused mha24k ring (step 0 writes, steps 1-3
    merge); one unfused ring (attention into the workspace plus the merge
    kernel).  Nothing is timed; the dispatch order is the record."""
    import torch

    import ring_blockwise_softmax_amd as ra
    from ring_blockwise_softmax_amd.workloads import Workload, WORKLOADS, make_inputs

    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    w = Workload("blk", 4, 32, 32, 128, 6000, 6000, 1, "contig", "bf16", 0.5, 9)
    q, k, v = make_inputs(w, device="cuda")
    out = torch.empty(4, 6000, 32, 128, device="cuda")
    lse = torch.empty(4, 32, 6000, device="cuda")
    for _ in range(2):
        ra.block_attn_fwd(q, k, v, out=out, lse=lse)
        torch.cuda.synchronize()
    q2, o2, l2 = q[:, :128].contiguous(), out[:, :128].contiguous(), lse[:, :, :128].contiguous()
    for _ in range(2):
        ra.block_attn_fwd(q2, k, v, out=o2, lse=l2)
        torch.cuda.synchronize()
    del q, k, v, out, lse, q2, o2, l2
    wm = WORKLOADS["mha24k"]
    q, k, v = make_inputs(wm, device="cuda")
    ra.RingRunner(q, k, v, wm.P, layout=wm.layout, fuse_merge=True).run()
    torch.cuda.synchronize()
    ra.RingRunner(q, k, v, wm.P, layout=wm.layout, fuse_merge=False).run()
    torch.cuda.synchronize()


def summarize_clock(samples):
    """Summary of gfx clock / power samples taken while the GPU was busy.

    samples: list of (per-XCD current gfx clocks in MHz, current socket power
    in W) tuples; entries that are not numbers ("N/A") are dropped.  The
    metrics table refreshes slower than it is sampled, so repeated values
    are kept as they come.
    """
    clocks, powers = [], []
    for xcd, power in samples:
        vals = [c for c in (xcd or []) if isinstance(c, (int, float))]
        if vals:
            clocks.append(sum(vals) / len(vals))
        if isinstance(power, (int, float)):
            powers.append(power)
    if not clocks:
        return None
    clocks.sort()
    out = {"sclk_mhz": round(clocks[len(clocks) // 2], 1),
           "sclk_mhz_range": [round(clocks[0], 1), round(clocks[-1], 1)],
           "samples": len(clocks)}
    if powers:
        powers.sort()
        out["socket_power_w"] = powers[len(powers) // 2]
    return out


def clock_telemetry(run_once, seconds=2.0, settle_s=0.5):
    """Sample the per-XCD gfx clocks and the socket power (amdsmi GPU
    metrics) while run_once() keeps the GPU busy for `seconds`; the first
    settle_s are not sampled (the table lags).  None if amdsmi is unusable."""
    import threading

    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception:
        return None
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        h = handles[0] if len(handles) == 1 else None
        if h is None:
            bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
            for c in handles:
                if bus is not None and int(amdsmi.amdsmi_get_gpu_device_bdf(c).split(":")[1], 16) == bus:
                    h = c
        if h is None:
            return None
        samples, stop = [], threading.Event()

        def sample():
            time.sleep(settle_s)
            while not stop.is_set():
                try:
                    m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                except Exception:
                    return
                samples.append((m.get("current_gfxclks"), m.get("current_socket_power")))
                stop.wait(0.05)

        th = threading.Thread(target=sample, daemon=True)
        t0 = time.perf_counter()
        th.start()
        while time.perf_counter() - t0 < seconds:
            for _ in range(5):
                run_once()
            torch.cuda.synchronize()
        stop.set()
        th.join()
        res = summarize_clock(samples)
        if res is not None:
            res["source"] = "amdsmi GPU metrics, sampled every 50 ms over %.1f s of steps" % (seconds - settle_s)
        return res
    except Exception:
        return None
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def mfma_ceiling(grid=2048, iters=2000):
    """The attention kernel's matrix instruction alone (libra_probe.so):
    TFLOP/s of v_mfma_f32_32x32x16_bf16 on random bf16 operands, with the
    clock and power it ran at, and the same loop on zero operands.  On
    random data the part cannot sustain its nominal clock, so this is the
    practical ceiling of a bf16 MFMA kernel on such inputs."""
    import ctypes

    import torch

    try:
        lib = ctypes.CDLL(os.path.join(ROOT, "ring_blockwise_softmax_amd", "libra_probe.so"))
    except OSError:
        return None  # probe library not built
    g = torch.Generator(device="cuda").manual_seed(1)
    src = (torch.randn(1024 * 8, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    sink = torch.empty(grid * 256, device="cuda")
    stream = torch.cuda.current_stream()
    flops = grid * 4 * iters * 8 * 2 * 32 * 32 * 16

    def make(zero):
        def run():
            rc = lib.ra_probe_mfma_loop(zero, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(sink.data_ptr()),
                                        grid, iters, ctypes.c_void_p(stream.cuda_stream))
            if rc:
                raise RuntimeError("MFMA probe launch failed (%d)" % rc)
        return run

    def rate(run, n=40):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        return flops / (e0.elapsed_time(e1) / n / 1e3) / 1e12

    out = {"kind": "v_mfma_f32_32x32x16_bf16 alone, operands cycling through random bf16 registers"}
    run = make(0)
    clock = clock_telemetry(run)          # also brings the part to its sustained clock
    out["tflops"] = round(rate(run), 1)
    if clock:
        out["sclk_mhz"], out["socket_power_w"] = clock["sclk_mhz"], clock.get("socket_power_w")
    zrun = make(1)
    for _ in range(100):
        zrun()
    out["zero_operands_tflops"] = round(rate(zrun), 1)
    return out


def f32_path_bench(steps=3):
    """The headline shape on the fp32 exact path (fp32 inputs, fp32 MFMA):
    the full fused ring, end to end and per attention launch, against the
    fp32 MFMA peak."""
    import torch

    import ring_blockwise_softmax_amd as ra
    from ring_blockwise_softmax_amd.workloads import make_inputs

    w = select_workload("mha24k", "f32")
    q, k, v = make_inputs(w, device="cuda")
    runner = ra.RingRunner(q, k, v, w.P, layout=w.layout, fuse_merge=True)
    for _ in range(2):
        runner.run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        runner.run()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    ra.profile_enable(True)
    for _ in range(steps):
        runner.run()
    prof = ra.profile_read()
    ra.profile_enable(False)
    n, ms = prof["attn"]
    flops = flops_of(w)
    per_launch = flops / (n / steps)
    achieved = per_launch / (ms / n / 1e3) / 1e12
    del q, k, v, runner
    torch.cuda.empty_cache()
    return {
        "workload": f"{w.name}: the headline shape with fp32 inputs (kernel attn_fwd_f32<{w.head_dim}>, fused merge)",
        "steps": steps,
        "ms_per_step": round(ms_step, 3),
        "tflops": round(flops / (ms_step / 1e3) / 1e12, 2),
        "avg_launch_ms": round(ms / n, 3),
        "achieved": round(achieved, 2),
        "peak": PEAK_F32_MFMA_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_F32_MFMA_TFLOPS, 4),
    }


def merge_bench(steps=10):
    """Standalone merge at the GQA 1M-token rank-share shape (>= 2 GB)."""
    import torch

    import ring_blockwise_softmax_amd as ra

    B, S, H, D = 1, 131072, 32, 128
    g = torch.Generator(device="cuda").manual_seed(44)
    out = torch.randn(B, S, H, D, device="cuda", generator=g)
    bout = torch.randn(B, S, H, D, device="cuda", generator=g)
    lse = torch.randn(B, H, S, device="cuda", generator=g)
    blse = torch.randn(B, H, S, device="cuda", generator=g)
    for _ in range(3):
        ra.merge(out, lse, bout, blse)
    torch.cuda.synchronize()
    ra.profile_enable(True)
    for _ in range(steps):
        ra.merge(out, lse, bout, blse)
    prof = ra.profile_read()
    ra.profile_enable(False)
    n, ms = prof["merge"]
    per = ms / n
    nbytes = B * S * H * (3 * 4 * D + 12)
    # plain device copy of the same byte count for reference
    src = torch.empty(nbytes // 2, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / steps
    del out, bout, lse, blse, src, dst
    torch.cuda.empty_cache()
    return {
        "shape": f"B{B} S{S} H{H} d{D} fp32",
        "bytes": nbytes,
        "ms": per,
        "achieved_GBs": nbytes / per / 1e6,
        "peak_GBs": PEAK_HBM_GBS,
        "frac": nbytes / per / 1e6 / PEAK_HBM_GBS,
        "copy_GBs": nbytes / copy_ms / 1e6,
        "step_shape": merge_step_bench(),
    }


def merge_step_bench(steps=12, sets=4):
    """Standalone merge at the 24k MHA step shape (all ranks' rows of one
    ring step: 1.19 GB, 297 MB per rank), cycling through `sets` buffer sets
    so that one call's operands are not still cached from the previous call."""
    import torch

    import ring_blockwise_softmax_amd as ra

    B, S, H, D = 1, 24000, 32, 128
    g = torch.Generator(device="cuda").manual_seed(45)
    bufs = [(torch.randn(B, S, H, D, device="cuda", generator=g), torch.randn(B, H, S, device="cuda", generator=g),
             torch.randn(B, S, H, D, device="cuda", generator=g), torch.randn(B, H, S, device="cuda", generator=g))
            for _ in range(sets)]
    for i in range(sets):
        ra.merge(*bufs[i])
    torch.cuda.synchronize()
    ra.profile_enable(True)
    for i in range(steps):
        ra.merge(*bufs[i % sets])
    prof = ra.profile_read()
    ra.profile_enable(False)
    n, ms = prof["merge"]
    per = ms / n
    nbytes = B * S * H * (3 * 4 * D + 12)
    del bufs
    torch.cuda.empty_cache()
    return {"shape": f"B{B} S{S} H{H} d{D} fp32, {sets} rotating buffer sets", "bytes": nbytes, "ms": per,
            "achieved_GBs": nbytes / per / 1e6, "frac": nbytes / per / 1e6 / PEAK_HBM_GBS}


def time_runner(runner, steps, warmup=None):
    """Warm-up (a fixed count, or at least 3 steps and 0.3 s so the clocks
    settle on short workloads too), then three timed regions of `steps` steps:
    the steps alone between two events (ms_step), the same steps with the
    library's event pair around every kernel launch (per-kernel times), and
    one event pair per step (the spread)."""
    import torch

    import ring_blockwise_softmax_amd as ra

    if warmup is not None:
        for _ in range(warmup):
            runner.run()
        torch.cuda.synchronize()
    else:
        warmup, t0 = 0, time.perf_counter()
        while warmup < 3 or time.perf_counter() - t0 < 0.3:
            runner.run()
            warmup += 1
            if warmup % 3 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        runner.run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    ra.profile_enable(True)
    for _ in range(steps):
        runner.run()
    torch.cuda.synchronize()
    prof = ra.profile_read()
    ra.profile_enable(False)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        runner.run()
        b.record(stream)
    torch.cuda.synchronize()
    return {"warmup": warmup, "steps": steps, "ms_step": ms_step,
            "per_step": sorted(a.elapsed_time(b) for a, b in evs), "prof": prof}


def roofline_of(w, rank, elem_size, tm):
    """The attention kernel against its roofline: algorithmic flops per launch
    over the average launch time (MFMA peak of the input dtype), or for the
    decode layout the K/V (+Q) bytes per launch over it (HBM peak)."""
    n_attn, attn_ms = tm["prof"]["attn"]
    launches_per_step = n_attn / tm["steps"]
    attn_avg_ms = attn_ms / n_attn
    flops_per_launch = flops_of(w, rank) / launches_per_step
    if w.layout == "kv_sharded":
        kv_bytes = 2 * w.batch * w.seq_k * w.heads_kv * w.head_dim * elem_size
        q_bytes = w.batch * w.seq_q * w.heads_q * w.head_dim * elem_size
        bytes_per_launch = (kv_bytes + q_bytes) / launches_per_step
        roof = {"bound": "hbm", "achieved": round(bytes_per_launch / (attn_avg_ms / 1e3) / 1e9, 2),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "algorithmic_bytes_per_launch": bytes_per_launch}
    else:
        roof = {"bound": "mfma", "achieved": round(flops_per_launch / (attn_avg_ms / 1e3) / 1e12, 2),
                "peak": peak_tflops(w), "unit": "TFLOP/s", "flops_per_launch": flops_per_launch}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    return roof, launches_per_step, attn_avg_ms


def other_workloads(names=("mha24k@0", "zigzag24k", "zigzag24k@0", "gqa1m", "mqa_decode", "prefill_chunk")):
    """The other configurations, each as it is run by --workload NAME (default
    rank, Ring order, fused; NAME@R: --workload NAME --rank R, one rank's
    share), in a compact record: end-to-end rate and the attention kernel
    against its roofline."""
    import torch

    import ring_blockwise_softmax_amd as ra
    from ring_blockwise_softmax_amd.workloads import make_inputs

    res = {}
    for key in names:
        name, _, r = key.partition("@")
        w = select_workload(name)
        rank = int(r) if r else w.rank
        q, k, v = make_inputs(w, device="cuda")
        runner = ra.RingRunner(q, k, v, w.P, layout=w.layout, rank=rank, fuse_merge=True)
        steps = 2 if name == "gqa1m" else 10
        tm = time_runner(runner, steps, 1 if name == "gqa1m" else None)
        roof, launches, avg_ms = roofline_of(w, rank, q.element_size(), tm)
        res[key] = {
            "workload": f"B{w.batch} Hq{w.heads_q}/Hkv{w.heads_kv} d{w.head_dim} Sq{w.seq_q} Sk{w.seq_k} "
                        f"P={w.P} ({w.layout}), {'all ranks' if rank < 0 else f'rank {rank}'}",
            "steps": steps, "warmup": tm["warmup"],
            "ms_per_step": round(tm["ms_step"], 4),
            "tflops": round(flops_of(w, rank) / (tm["ms_step"] / 1e3) / 1e12, 2),
            "kernel": {"launches_per_step": launches, "avg_launch_ms": round(avg_ms, 4),
                       **{k_: v_ for k_, v_ in roof.items() if k_ in ("bound", "achieved", "peak", "unit", "frac")}},
        }
        del q, k, v, runner
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 3 and at least 0.3 s of steps, "
                         "so the clocks settle on short workloads too)")
    ap.add_argument("--workload", default="mha24k")
    ap.add_argument("--dtype", default=None, choices=["bf16", "f32"],
                    help="run the workload's shape in this input dtype (f32: the exact path)")
    ap.add_argument("--order", default="ring", choices=["ring", "tokenring"])
    ap.add_argument("--unfused", action="store_true", help="separate merge kernel")
    ap.add_argument("--rank", type=int, default=None, help="emulate one rank's share only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-merge", action="store_true")
    ap.add_argument("--no-f32", action="store_true", help="skip the fp32 exact-path run of the headline shape")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the compact runs of the other configurations after the headline")
    ap.add_argument("--no-clock", action="store_true", help="skip the clock / power sampling")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the MFMA-only ceiling measurement")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--oracle-table", action="store_true",
                    help="only time the CPU oracle per configuration beside the GPU (one JSON line each)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only run the fixed launch sequence used for per-dispatch counter runs")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the ring is emulated in one device's memory; "
              "--gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)

    if args.oracle_table:
        oracle_table()
        return
    if args.traffic_probe:
        traffic_probe()
        return

    import torch

    import ring_blockwise_softmax_amd as ra
    from ring_blockwise_softmax_amd.workloads import make_inputs

    w = select_workload(args.workload, args.dtype)
    rank = w.rank if args.rank is None else args.rank
    q, k, v = make_inputs(w, device="cuda")
    runner = ra.RingRunner(q, k, v, w.P, layout=w.layout, order=args.order, rank=rank,
                           fuse_merge=not args.unfused)
    tm = time_runner(runner, args.steps, args.warmup)
    args.warmup = tm["warmup"]
    ms_step, per_step = tm["ms_step"], tm["per_step"]
    total_flops = flops_of(w, rank)
    tflops = total_flops / (ms_step / 1e3) / 1e12
    roof, launches_per_step, attn_avg_ms = roofline_of(w, rank, q.element_size(), tm)
    peak = peak_tflops(w)

    rec = {
        "metric": "attention TFLOP/s + % bf16 MFMA peak at S=24000, H=32, d=128, 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1)*%g Q/K/V)" % w.std,
        "config": {
            "workload": f"{w.name}: B{w.batch} Hq{w.heads_q}/Hkv{w.heads_kv} d{w.head_dim} "
                        f"S{w.seq_q} over P={w.P} ({w.layout}), {'all ranks' if rank < 0 else f'rank {rank}'}",
            "global_batch": w.batch,
            "seq_len": w.seq_q,
            "P": w.P,
            "layout": w.layout,
            "order": args.order,
            "fuse_merge": not args.unfused,
            "flops_per_step": total_flops,
            "parallelism": "single GPU, ring emulated in device memory",
        },
        "pct_peak": round(100.0 * tflops / peak, 2),
        "roofline": {
            "bound": roof["bound"],
            "kernel": ("attn_fwd_bf16<%d>" % w.head_dim if w.dtype == "bf16" else "attn_fwd_f32<%d>" % w.head_dim)
                      + ("" if args.unfused
                         else " (partials for the gather-merge)" if w.layout.startswith("kv_sharded")
                         else " (fused merge epilogue)"),
            "achieved": roof["achieved"],
            "peak": roof["peak"],
            "unit": roof["unit"],
            "frac": roof["frac"],
            "traffic": measured_traffic(w.name),
            "launches_per_step": launches_per_step,
            "avg_launch_ms": round(attn_avg_ms, 4),
            **{k_: v_ for k_, v_ in roof.items() if k_ in ("flops_per_launch", "algorithmic_bytes_per_launch")},
        },
        "step_ms": {"min": round(per_step[0], 4), "median": round(per_step[len(per_step) // 2], 4),
                    "max": round(per_step[-1], 4)},
        "seed": w.seed,
        "hip": torch.version.hip,
    }
    # Region 4 (not timed): clocks and power while the same steps run.
    if not args.no_clock:
        rec["clock"] = clock_telemetry(runner.run)
        if rec["clock"] and rec["roofline"]["unit"] == "TFLOP/s":
            # the same kernel against the MFMA peak at the clock it ran at
            rec["roofline"]["frac_at_sclk"] = round(
                roof["achieved"] / (roof["peak"] * rec["clock"]["sclk_mhz"] / 2400.0), 4)
    if not args.no_ceiling and rec["roofline"]["unit"] == "TFLOP/s" and w.dtype == "bf16":
        ceiling = mfma_ceiling()
        if ceiling:
            rec["roofline"]["ceiling"] = ceiling
            rec["roofline"]["frac_of_ceiling"] = round(roof["achieved"] / ceiling["tflops"], 4)
    if args.calib_copy:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_merge:
        rec["merge"] = merge_bench()
    if not args.no_f32 and args.workload == "mha24k" and w.dtype == "bf16":
        rec["f32_path"] = f32_path_bench()
    if not args.no_others and args.workload == "mha24k" and w.dtype == "bf16":
        rec["other_workloads"] = other_workloads()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, runner.out, runner.lse, rank)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
