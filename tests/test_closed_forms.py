"""Pin the oracle with closed forms and an independent library routine.

* Q = 0: every visible key gets the same weight, so lse_i = ln |J(i)| and out_i
  is the mean of the visible V rows (causal: ln(i+1) and a prefix mean).
* V constant per K/V head: out equals that head's constant, which pins the
  grouped-query head map (query head h reads K/V head floor(h / group)).
* One-hot V: out is the weight vector, which pins which keys contributed.
* A single key: out = v_0 and lse = its scaled score.
* torch's CPU scaled-dot-product attention in fp64 (with GQA) for ``out``.
"""

import math

import numpy as np
import pytest

from oracle import attention


def test_zero_queries_uniform_weights_noncausal():
    rng = np.random.default_rng(1)
    B, Sq, Sk, Hq, Hkv, d = 2, 5, 37, 4, 2, 8
    q = np.zeros((B, Sq, Hq, d))
    k = rng.standard_normal((B, Sk, Hkv, d))
    v = rng.standard_normal((B, Sk, Hkv, d))
    o, l = attention(q, k, v)
    assert np.max(np.abs(l - math.log(Sk))) < 1e-13
    for h in range(Hq):
        g = h // (Hq // Hkv)
        mean = v[:, :, g, :].mean(axis=1)          # [B, d]
        assert np.max(np.abs(o[:, :, h, :] - mean[:, None, :])) < 1e-13


def test_zero_queries_causal_prefix_mean():
    rng = np.random.default_rng(2)
    B, S, H, d = 1, 40, 2, 4
    q = np.zeros((B, S, H, d))
    k = rng.standard_normal((B, S, H, d))
    v = rng.standard_normal((B, S, H, d))
    o, l = attention(q, k, v, causal=True)
    i = np.arange(S)
    assert np.max(np.abs(l - np.log(i + 1)[None, None, :])) < 1e-13
    prefix_mean = np.cumsum(v, axis=1) / (i + 1)[None, :, None, None]
    assert np.max(np.abs(o - prefix_mean)) < 1e-13


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 2), (4, 1), (32, 8)])
def test_constant_v_pins_head_map(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    B, S, d = 1, 9, 4
    q = rng.standard_normal((B, S, Hq, d)) * 3
    k = rng.standard_normal((B, S, Hkv, d)) * 3
    const = np.arange(Hkv, dtype=np.float64)[:, None] * 10.0 + np.arange(d)[None, :]
    v = np.broadcast_to(const[None, None], (B, S, Hkv, d)).copy()
    o, _ = attention(q, k, v, causal=True)
    group = Hq // Hkv
    for h in range(Hq):
        assert np.max(np.abs(o[0, :, h, :] - const[h // group])) < 1e-12


def test_one_hot_v_gives_weights():
    special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(4)
    S, d = 6, 8
    q = rng.standard_normal((1, S, 1, d)) * 2
    k = rng.standard_normal((1, S, 1, d)) * 2
    v = np.zeros((1, S, 1, d))
    v[0, np.arange(S), 0, np.arange(S)] = 1.0          # key j -> unit vector e_j
    o, l = attention(q, k, v, causal=True)
    scores = (q[0, :, 0, :] @ k[0, :, 0, :].T) / math.sqrt(d)
    scores = np.where(np.tril(np.ones((S, S), bool)), scores, -np.inf)
    w = special.softmax(scores, axis=1)
    assert np.max(np.abs(o[0, :, 0, :S] - w)) < 1e-13
    assert np.all(o[0, :, 0, S:] == 0.0)
    assert np.max(np.abs(l[0, 0] - special.logsumexp(scores, axis=1))) < 1e-13


def test_single_key():
    rng = np.random.default_rng(5)
    d = 16
    q = rng.standard_normal((1, 3, 2, d))
    k = rng.standard_normal((1, 1, 2, d))
    v = rng.standard_normal((1, 1, 2, d))
    o, l = attention(q, k, v)
    for h in range(2):
        assert np.max(np.abs(o[0, :, h] - v[0, 0, h][None])) < 1e-15
        s = q[0, :, h] @ k[0, 0, h] / math.sqrt(d)
        assert np.max(np.abs(l[0, h] - s)) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (4, 1)])
def test_torch_sdpa_fp64_cross_check(causal, Hq, Hkv):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    g = torch.Generator().manual_seed(123)
    B, S, d = 2, 33, 16
    q = torch.randn(B, S, Hq, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, S, Hkv, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, S, Hkv, d, generator=g, dtype=torch.float64)
    ref = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2),
                                         is_causal=causal, enable_gqa=True).transpose(1, 2)
    o, _ = attention(q.numpy(), k.numpy(), v.numpy(), causal=causal)
    assert np.max(np.abs(o - ref.numpy())) < 1e-12
