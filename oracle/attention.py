"""One-shot softmax attention in fp64 (test infrastructure; see package doc).

Definition followed (the plain result the method reaches exactly; TokenRing
review, "What carries the argument" and "Assumptions" -- the merge reproduces
standard attention; Ring Attention record -- no approximation):

    g(h)   = floor(h / (Hq / Hkv))                 K/V head of query head h
    s_ij   = tau * <q[b,i,h,:], k[b,j,g,:]>,        tau = 1/sqrt(d)
    J(i)   = all j                                  (non-causal)
           = { j : kpos[j] <= qpos[i] }             (causal, global positions)
    lse_i  = ln sum_{j in J(i)} exp(s_ij)           (natural log)
    out_i  = sum_{j in J(i)} exp(s_ij - lse_i) v[b,j,g,:]
    J(i) = {}  ->  lse_i = -inf, out_i = 0

The grouped-query head map (contiguous groups) is the plain reading of the
TokenRing review's remark that grouped- and multi-query attention keep working
("If this is right", with its references to MQA and GQA).

Layouts: q is [B, Sq, Hq, d], k and v are [B, Sk, Hkv, d] (token-major, d
last), out is [B, Sq, Hq, d] and lse is [B, Hq, Sq].  Inputs of any float
dtype (including torch bfloat16 tensors) are upcast to fp64 exactly.
"""

from __future__ import annotations

import math

import numpy as np

ROW_CHUNK = 512


def _as_f64(x) -> np.ndarray:
    """Exact upcast to a float64 numpy array (accepts numpy or torch CPU)."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64, copy=False)
    # torch tensor: bf16 -> fp32 -> fp64 are both exact widenings.
    import torch  # local: the oracle itself never needs torch otherwise

    t = x.detach().to("cpu")
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.to(torch.float32)
    return t.to(torch.float64).numpy()


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """K/V head read by query head ``h``: contiguous groups of Hq/Hkv heads."""
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (hq // hkv)


def attention(q, k, v, causal: bool = False, q_pos=None, k_pos=None,
              rows=None, scale: float | None = None):
    """Exact softmax attention and its natural-log row log-sum-exp, in fp64.

    Args:
      q: [B, Sq, Hq, d];  k, v: [B, Sk, Hkv, d].
      causal: if True, key j is visible to query i iff k_pos[j] <= q_pos[i].
      q_pos, k_pos: global token positions of the rows of q and k (default
        0..Sq-1 and 0..Sk-1).  They only matter when ``causal`` is True.
      rows: optional 1-D integer array of query indices to evaluate (the
        result then has len(rows) in place of Sq).
      scale: softmax scale, default 1/sqrt(d).

    Returns:
      (out, lse): out [B, R, Hq, d] fp64, lse [B, Hq, R] fp64, R = #rows.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Sq, Hq, d = q.shape
    Bk, Sk, Hkv, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k, v")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    tau = 1.0 / math.sqrt(d) if scale is None else float(scale)
    q_pos = np.arange(Sq, dtype=np.int64) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    k_pos = np.arange(Sk, dtype=np.int64) if k_pos is None else np.asarray(k_pos, dtype=np.int64)
    rows = np.arange(Sq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]

    out = np.zeros((B, R, Hq, d), dtype=np.float64)
    lse = np.full((B, Hq, R), -np.inf, dtype=np.float64)
    if Sk == 0 or R == 0:
        return out, lse

    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kg = k[b, :, g, :]            # [Sk, d]
            vg = v[b, :, g, :]            # [Sk, d]
            for r0 in range(0, R, ROW_CHUNK):
                rr = rows[r0:r0 + ROW_CHUNK]
                qi = q[b, rr, h, :]       # [r, d]
                s = tau * (qi @ kg.T)     # [r, Sk]
                if causal:
                    visible = k_pos[None, :] <= q_pos[rr][:, None]
                    s = np.where(visible, s, -np.inf)
                m = np.max(s, axis=1)     # [r]
                empty = ~np.isfinite(m)
                m_safe = np.where(empty, 0.0, m)
                e = np.exp(s - m_safe[:, None])
                z = np.sum(e, axis=1)
                with np.errstate(divide="ignore"):
                    row_lse = m_safe + np.log(z)
                row_lse = np.where(empty, -np.inf, row_lse)
                w = np.where(empty[:, None], 0.0, np.exp(s - np.where(empty, 0.0, row_lse)[:, None]))
                out[b, r0:r0 + len(rr), h, :] = w @ vg
                lse[b, h, r0:r0 + len(rr)] = row_lse
    return out, lse
