"""Pins for the oracle's greedy prefix acceptance: hand-derived golden cases,
closed forms, the losslessness invariant and exhaustive enumeration."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import verify

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "verify_cases.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_golden_cases(case):
    t = np.array([case["target"]])
    d = np.array([case["drafts"]], dtype=np.int64).reshape(1, len(case["drafts"]))
    acc, out = verify.greedy_verify(t, d, case["vocab"])
    assert acc[0] == case["accepted_len"]
    assert out[0].tolist() == case["out_tokens"]
    assert verify.verified_tokens(acc) == case["accepted_len"] + 1


def test_closed_forms_batch():
    k, v = 15, 1000
    rng = np.random.default_rng(41)
    t = rng.integers(0, v, size=(6, k + 1))
    d = np.empty((6, k), dtype=np.int64)
    d[0] = t[0, :k]                                  # all correct -> K
    d[1] = t[1, :k]; d[1, 0] = (t[1, 0] + 1) % v      # first wrong -> 0
    d[2] = t[2, :k]; d[2, 7] = -1                    # sentinel at 7 -> 7
    d[3] = -1                                        # all sentinels -> 0
    d[4] = t[4, :k]; d[4, 14] = (t[4, 14] + 1) % v    # last wrong -> 14
    d[5] = t[5, :k]; d[5, 3] = v + 3                 # out of range at 3 -> 3
    acc, out = verify.greedy_verify(t, d, v)
    assert acc.tolist() == [15, 0, 7, 0, 14, 3]
    for b in range(6):
        a = acc[b]
        assert np.array_equal(out[b, :a + 1], t[b, :a + 1])     # lossless invariant
        assert np.all(out[b, a + 1:] == -1)
    assert verify.verified_tokens(acc) == 16 + 1 + 8 + 1 + 15 + 4


def test_k_zero():
    acc, out = verify.greedy_verify(np.array([[7], [2]]), np.zeros((2, 0), np.int64), 10)
    assert acc.tolist() == [0, 0]
    assert out.tolist() == [[7], [2]]


def _spelled_out(t, d, v):
    """a = the largest j such that every draft before j is in range and equal to its target."""
    k = len(d)
    best = 0
    for j in range(k + 1):
        if all(0 <= d[i] < v and d[i] == t[i] for i in range(j)):
            best = j
    return best


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_exhaustive_small(k):
    v = 3
    ts = list(itertools.product(range(v), repeat=k + 1))
    ds = list(itertools.product([-1, 0, 1, 2], repeat=k))
    rng = np.random.default_rng(k)
    # every draft vector against a sample of target vectors (all of them for k <= 3)
    tsel = ts if k <= 3 else [ts[i] for i in rng.choice(len(ts), 24, replace=False)]
    tt = np.array([t for t in tsel for _ in ds])
    dd = np.array([d for _ in tsel for d in ds])
    acc, out = verify.greedy_verify(tt, dd, v)
    for i in range(len(tt)):
        a = _spelled_out(tt[i], dd[i], v)
        assert acc[i] == a
        assert out[i].tolist() == list(tt[i][:a + 1]) + [-1] * (k - a)
