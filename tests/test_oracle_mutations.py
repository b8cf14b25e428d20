"""Plant plausible mistakes in the oracle (on the CPU) and check a pin fails.

This shows the pins discriminate: a wrong grouped-query head map, a dropped
softmax scale, a log-base slip, a flipped sigma argument or a sequential
(lse-first) reading of the merge rule would each be caught.
"""

import json
import math
import os

import numpy as np
import pytest

import importlib
from oracle import attention, merge_stable

oatt = importlib.import_module("oracle.attention")
from tests.test_oracle_bruteforce import brute_force

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_wrong_head_map_is_caught(monkeypatch):
    rng = np.random.default_rng(0)
    Hq, Hkv, d, S = 4, 2, 4, 6
    q = rng.standard_normal((1, S, Hq, d))
    k = rng.standard_normal((1, S, Hkv, d))
    const = np.array([[1.0] * d, [5.0] * d])
    v = np.broadcast_to(const[None, None], (1, S, Hkv, d)).copy()
    monkeypatch.setattr(oatt, "kv_head_of", lambda h, hq, hkv: h % hkv)
    o, _ = oatt.attention(q, k, v)
    errs = [np.max(np.abs(o[0, :, h] - const[h // 2])) for h in range(Hq)]
    assert max(errs) > 1.0


def test_dropped_scale_and_log_base_are_caught():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 5, 1, 8))
    k = rng.standard_normal((1, 7, 1, 8))
    v = rng.standard_normal((1, 7, 1, 8))
    o_b, l_b = brute_force(q, k, v, False, list(range(5)), list(range(7)))
    o, l = attention(q, k, v, scale=1.0)                 # tau dropped
    assert np.max(np.abs(l - l_b)) > 1e-3
    o, l = attention(q, k, v)
    assert np.max(np.abs(l / math.log(2) - l_b)) > 1e-3  # lse in log2 units


def _merge_lse_first(out, lse, bout, blse):
    # Wrong reading: update lse first, then use the new lse in the out update.
    new_lse = lse - np.log(1 / (1 + np.exp(-(lse - blse))))
    w = 1 / (1 + np.exp(-(blse - new_lse)))
    return out - w[..., None] * (out - bout), new_lse


def _merge_flipped_sigma(out, lse, bout, blse):
    w = 1 / (1 + np.exp(-(lse - blse)))
    return out - w[..., None] * (out - bout), lse - np.log(1 / (1 + np.exp(-(lse - blse))))


@pytest.mark.parametrize("bad", [_merge_lse_first, _merge_flipped_sigma])
def test_wrong_merge_readings_fail_golden(bad):
    with open(os.path.join(GOLDEN, "merge_cases.json")) as f:
        cases = json.load(f)["cases"]
    caught = False
    for c in cases[:3]:
        o, l = bad(np.array([c["out"]]), np.array([float(c["lse"])]),
                   np.array([c["block_out"]]), np.array([float(c["block_lse"])]))
        if np.max(np.abs(o[0] - c["new_out"])) > 1e-6 or abs(l[0] - float(c["new_lse"])) > 1e-6:
            caught = True
    assert caught
    # and the correct rule passes the same cases
    for c in cases[:3]:
        o, l = merge_stable(np.array([c["out"]]), np.array([float(c["lse"])]),
                            np.array([c["block_out"]]), np.array([float(c["block_lse"])]))
        assert np.max(np.abs(o[0] - c["new_out"])) < 1e-12
