"""Pin the fp64 oracle against brute force with scalar Python arithmetic.

The brute force below is written independently of ``oracle.attention``: plain
Python floats, ``math.exp`` and ``math.fsum`` (exactly rounded sums), one
(query, head) at a time, straight from the definition of softmax attention
with a natural-log log-sum-exp.  A dropped scale, a wrong GQA map, a wrong
mask convention or a log base other than e makes the comparison fail.
"""

import math

import numpy as np
import pytest

from oracle import attention


def brute_force(q, k, v, causal, qpos, kpos):
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    group = Hq // Hkv
    tau = 1.0 / math.sqrt(d)
    out = [[[[0.0] * d for _ in range(Hq)] for _ in range(Sq)] for _ in range(B)]
    lse = [[[-math.inf] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for i in range(Sq):
            for h in range(Hq):
                g = h // group
                keys = [j for j in range(Sk) if (not causal) or kpos[j] <= qpos[i]]
                if not keys:
                    continue
                s = {}
                for j in keys:
                    s[j] = tau * math.fsum(float(q[b, i, h, t]) * float(k[b, j, g, t]) for t in range(d))
                m = max(s.values())
                z = math.fsum(math.exp(s[j] - m) for j in keys)
                L = m + math.log(z)
                lse[b][h][i] = L
                for t in range(d):
                    out[b][i][h][t] = math.fsum(math.exp(s[j] - L) * float(v[b, j, g, t]) for j in keys)
    return np.array(out), np.array(lse)


CASES = [
    # (B, Sq, Sk, Hq, Hkv, d, causal)
    (1, 5, 7, 1, 1, 4, False),
    (2, 6, 6, 4, 4, 8, True),
    (1, 9, 9, 4, 2, 4, True),
    (1, 3, 11, 4, 1, 8, False),
    (1, 16, 16, 4, 1, 8, True),
    (2, 4, 13, 2, 2, 2, False),
]


@pytest.mark.parametrize("B,Sq,Sk,Hq,Hkv,d,causal", CASES)
def test_oracle_matches_brute_force(B, Sq, Sk, Hq, Hkv, d, causal):
    rng = np.random.default_rng(1000 + Sq * 31 + Sk)
    q = rng.standard_normal((B, Sq, Hq, d)) * 1.5
    k = rng.standard_normal((B, Sk, Hkv, d)) * 1.5
    v = rng.standard_normal((B, Sk, Hkv, d))
    qpos = np.arange(Sq) + (Sk - Sq)          # bottom-right aligned positions
    kpos = np.arange(Sk)
    o_ref, l_ref = brute_force(q, k, v, causal, qpos, kpos)
    o, l = attention(q, k, v, causal=causal, q_pos=qpos, k_pos=kpos)
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.max(np.abs(l - l_ref)) < 1e-12


def test_oracle_row_subset_matches_full():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 40, 4, 8))
    k = rng.standard_normal((2, 40, 2, 8))
    v = rng.standard_normal((2, 40, 2, 8))
    rows = np.array([0, 3, 17, 39, 5])
    o_full, l_full = attention(q, k, v, causal=True)
    o_sub, l_sub = attention(q, k, v, causal=True, rows=rows)
    assert np.array_equal(o_sub, o_full[:, rows])
    assert np.array_equal(l_sub, l_full[:, :, rows])


def test_oracle_empty_rows_are_identity():
    # Query positions before every key: no visible key -> (0, -inf).
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 3, 2, 4))
    k = rng.standard_normal((1, 5, 2, 4))
    v = rng.standard_normal((1, 5, 2, 4))
    o, l = attention(q, k, v, causal=True, q_pos=np.array([-3, -1, 2]), k_pos=np.arange(5))
    assert np.all(o[:, :2] == 0.0) and np.all(np.isneginf(l[:, :, :2]))
    assert np.all(np.isfinite(l[:, :, 2]))
    o_b, l_b = brute_force(q, k, v, True, [-3, -1, 2], list(range(5)))
    assert np.max(np.abs(o - o_b)) < 1e-12


def test_oracle_bf16_inputs_are_upcast_exactly():
    torch = pytest.importorskip("torch")
    g = torch.Generator().manual_seed(11)
    q = torch.randn(1, 6, 2, 8, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 6, 2, 8, generator=g).to(torch.bfloat16)
    v = torch.randn(1, 6, 2, 8, generator=g).to(torch.bfloat16)
    o, l = attention(q, k, v, causal=True)
    qn, kn, vn = (t.float().double().numpy() for t in (q, k, v))
    o_b, l_b = brute_force(qn, kn, vn, True, list(range(6)), list(range(6)))
    assert np.max(np.abs(o - o_b)) < 1e-12
    assert np.max(np.abs(l - l_b)) < 1e-12
