"""Python entry points with the C ABI's names (marshalling only).

block_attn_fwd  -- one query block against one K/V block -> (block_out, block_lse)
block_attn_fwd_noalloc -- the same into caller-provided outputs, no allocation
merge           -- fold a partial into the running (out, lse), in place
ring_forward    -- the emulated P-step ring (Ring Attention / TokenRing order,
                   contiguous or zigzag causal partition)
ring_plan       -- the host-side work list of the ring

Tensors: q [B, Sq, Hq, d], k/v [B, Sk, Hkv, d] (bf16 or fp32, d contiguous),
out [B, Sq, Hq, d] fp32, lse [B, Hq, Sq] fp32, all on one GPU.  Work is
enqueued on ``stream`` (default: torch's current stream); nothing
synchronises.
"""

from __future__ import annotations

import ctypes

from . import _lib as L


def _empty_out(q):
    import torch

    B, S, H, D = q.shape
    out = torch.empty((B, S, H, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    return out, lse


def _workspace(nbytes, device):
    import torch

    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _on_one_gpu(*tensors):
    """The kernels dereference every data pointer on the device: refuse host
    tensors and tensors spread over several GPUs before anything is called."""
    devs = {t.device for t in tensors if t is not None}
    if any(d.type != "cuda" for d in devs):
        raise ValueError("tensors must be on a GPU device (got %s)" % sorted(str(d) for d in devs))
    if len(devs) > 1:
        raise ValueError("tensors must be on one GPU (got %s)" % sorted(str(d) for d in devs))


def _used_on(stream, *tensors):
    """Mark tensors allocated on torch's current stream as used by ``stream``.

    The kernels run on ``stream``; when that is not the current stream, the
    caching allocator must not hand these blocks to other work (e.g. after a
    temporary workspace is freed on return) before ``stream`` has finished.
    """
    import torch

    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def block_attn_workspace_bytes(q, k) -> int:
    tq, tk = L.bshd(q), L.bshd(k)
    return int(L.lib().ra_block_attn_workspace_bytes(ctypes.byref(tq), ctypes.byref(tk)))


def block_attn_fwd(q, k, v, mask="none", out=None, lse=None, workspace=None, stream=None):
    """block_out, block_lse of q against (k, v); mask: none | causal | causal_bottom_right."""
    _on_one_gpu(q, k, v, out, lse, workspace)
    lib = L.lib()
    if out is None or lse is None:
        out, lse = _empty_out(q)
    tq, tk, tv = L.bshd(q), L.bshd(k), L.bshd(v)
    to, tl = L.bshd(out), L.lse_desc(lse)
    if workspace is None:
        workspace = _workspace(block_attn_workspace_bytes(q, k), q.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    L.check(lib.ra_block_attn_fwd(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), L.MASKS[mask],
                                  ctypes.byref(to), ctypes.byref(tl), wptr, wbytes, L.stream_ptr(stream)))
    _used_on(stream, out, lse, workspace)
    return out, lse


def block_attn_fwd_noalloc(q, k, v, out, lse, mask="none", stream=None):
    """block_attn_fwd into caller-provided out/lse with no allocation at all:
    split-K partials use the library's static device scratch (calls that
    overlap in time on one GPU race; calls in one stream are ordered)."""
    _on_one_gpu(q, k, v, out, lse)
    lib = L.lib()
    tq, tk, tv = L.bshd(q), L.bshd(k), L.bshd(v)
    to, tl = L.bshd(out), L.lse_desc(lse)
    L.check(lib.ra_block_attn_fwd_noalloc(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), L.MASKS[mask],
                                          ctypes.byref(to), ctypes.byref(tl), L.stream_ptr(stream)))
    return out, lse


def merge(out, lse, block_out, block_lse, stream=None):
    """In place: (out, lse) <- sigma-rule merge with (block_out, block_lse)."""
    _on_one_gpu(out, lse, block_out, block_lse)
    lib = L.lib()
    to, tl = L.bshd(out), L.lse_desc(lse)
    tbo, tbl = L.bshd(block_out), L.lse_desc(block_lse)
    L.check(lib.ra_merge(ctypes.byref(to), ctypes.byref(tl), ctypes.byref(tbo), ctypes.byref(tbl),
                         L.stream_ptr(stream)))
    return out, lse


def _layout(layout, order, rank, fuse_merge, ws=None, ws_bytes=0):
    return L.RaLayout(L.LAYOUTS[layout], L.ORDERS[order], rank, 1 if fuse_merge else 0, ws, ws_bytes)


def ring_workspace_bytes(q, k, P, layout="contig", order="ring", rank=-1, fuse_merge=True) -> int:
    tq, tk = L.bshd(q), L.bshd(k)
    lay = _layout(layout, order, rank, fuse_merge)
    return int(L.lib().ra_ring_workspace_bytes(ctypes.byref(tq), ctypes.byref(tk), P, ctypes.byref(lay)))


class RingRunner:
    """Pre-marshalled ring_forward call (descriptors and workspace built once).

    Re-invoking ``run()`` repeats the exact same enqueue sequence; used by the
    benchmark so the timed loop contains only the library call.
    """

    def __init__(self, q, k, v, P, layout="contig", order="ring", rank=-1, fuse_merge=True,
                 out=None, lse=None, workspace=None):
        _on_one_gpu(q, k, v, out, lse, workspace)
        self.lib = L.lib()
        if out is None or lse is None:
            out, lse = _empty_out(q)
        self.out, self.lse = out, lse
        nbytes = ring_workspace_bytes(q, k, P, layout, order, rank, fuse_merge)
        if workspace is None:
            workspace = _workspace(nbytes, q.device)
        self.workspace = workspace
        wptr = workspace.data_ptr() if workspace is not None else None
        wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        self._keep = (q, k, v)
        self.tq, self.tk, self.tv = L.bshd(q), L.bshd(k), L.bshd(v)
        self.to, self.tl = L.bshd(out), L.lse_desc(lse)
        self.lay = _layout(layout, order, rank, fuse_merge, wptr, wbytes)
        self.P = P

    def run(self, stream=None):
        L.check(self.lib.ra_ring_forward(ctypes.byref(self.tq), ctypes.byref(self.tk), ctypes.byref(self.tv),
                                         self.P, ctypes.byref(self.lay), ctypes.byref(self.to),
                                         ctypes.byref(self.tl), L.stream_ptr(stream)))
        _used_on(stream, self.out, self.lse, self.workspace)
        return self.out, self.lse


def ring_forward(q, k, v, P, layout="contig", order="ring", rank=-1, fuse_merge=True,
                 out=None, lse=None, workspace=None, stream=None):
    """Exact attention through the emulated P-step ring; returns (out, lse).

    Rows not owned by ``rank`` (when rank >= 0) are left as they were in
    ``out``/``lse`` (uninitialised if those were allocated here).
    """
    r = RingRunner(q, k, v, P, layout, order, rank, fuse_merge, out, lse, workspace)
    return r.run(stream)


def ring_plan(Sq, Sk, P, layout="contig", order="ring", rank=-1):
    """The host-side work list as a list of dicts (no GPU needed)."""
    lib = L.lib()
    lay = _layout(layout, order, rank, True)
    n = lib.ra_ring_plan(Sq, Sk, P, ctypes.byref(lay), None, 0)
    if n < 0:
        raise ValueError(f"no ring plan for Sq={Sq} Sk={Sk} P={P} layout={layout} rank={rank}")
    arr = (L.RaPlanItem * max(n, 1))()
    if lib.ra_ring_plan(Sq, Sk, P, ctypes.byref(lay), arr, n) != n:
        raise RuntimeError("ring plan changed size between the count and the fill")
    items = []
    for it in arr[:n]:
        items.append({
            "step": it.step, "rank": it.rank, "q_start": it.q_start, "q_len": it.q_len, "q_pos0": it.q_pos0,
            "first": bool(it.first),
            "segs": [{"kv_start": it.seg[i].kv_start, "kv_len": it.seg[i].kv_len,
                      "causal": bool(it.seg[i].causal), "kv_rank": it.seg[i].kv_rank}
                     for i in range(it.nseg)],
        })
    return items


def profile_enable(on=True):
    L.check(L.lib().ra_profile_enable(1 if on else 0))


def profile_read():
    """{kind: (launches, total_ms)} since the last enable/read (synchronises)."""
    n = len(L.KERNEL_KINDS)
    cnt = (ctypes.c_int64 * n)()
    ms = (ctypes.c_double * n)()
    L.check(L.lib().ra_profile_read(cnt, ms, n))
    return {k: (int(cnt[i]), float(ms[i])) for i, k in enumerate(L.KERNEL_KINDS)}
