"""Pins for the recurrent-state commit oracle: closed forms of the gated delta
rule (no write keeps a decayed state; a full-strength write along a unit key
replaces that key's column; orthogonal keys write independent columns), the
accepted-length semantics (a + 1 updates, clamping, splitting the prefix),
and exact rationals on a tiny state."""
from fractions import Fraction

import numpy as np
import pytest

import gen
from oracle import gdn


def test_no_write_decays_the_state():
    rng = np.random.default_rng(1)
    S, k, v, _, _ = gen.gdn_inputs(rng, 1, 5, 2, 8, 6)
    alpha = np.full((1, 5, 2), 0.5, np.float32)
    beta = np.zeros((1, 5, 2), np.float32)
    for a in range(5):
        out = gdn.commit(S, k, v, alpha, beta, [a])
        assert np.allclose(out, S.astype(np.float64) * 0.5 ** (a + 1), rtol=0, atol=1e-15)


def test_full_write_along_unit_keys_replaces_columns():
    # alpha = 1, beta = 1, k_t = e_{j_t}: column j_t of S becomes v_t, the rest stays
    dk, dv = 6, 4
    S = np.arange(dv * dk, dtype=np.float64).reshape(1, 1, dv, dk)
    cols = [2, 5, 2, 0]
    T = len(cols)
    k = np.zeros((1, T, 1, dk))
    for t, j in enumerate(cols):
        k[0, t, 0, j] = 1.0
    v = np.arange(T * dv, dtype=np.float64).reshape(1, T, 1, dv) + 100
    ones = np.ones((1, T, 1))
    out = gdn.commit(S, k, v, ones, ones, [3])[0, 0]
    expect = S[0, 0].copy()
    for t, j in enumerate(cols):
        expect[:, j] = v[0, t, 0]
    assert np.array_equal(out, expect)


def test_accepted_length_counts_updates_and_clamps():
    rng = np.random.default_rng(2)
    S, k, v, al, be = gen.gdn_inputs(rng, 3, 6, 2, 8, 8)
    by_hand = S.astype(np.float64).copy()
    for b, a in enumerate([0, 5, 2]):
        for h in range(2):
            M = by_hand[b, h]
            for t in range(a + 1):
                M = gdn.gdn_update(M, k[b, t, h], v[b, t, h], al[b, t, h], be[b, t, h])
            by_hand[b, h] = M
    assert np.array_equal(gdn.commit(S, k, v, al, be, [0, 5, 2]), by_hand)
    # out-of-range accepted lengths clamp to [0, T - 1]
    assert np.array_equal(gdn.commit(S, k, v, al, be, [-4, 99, 2]), gdn.commit(S, k, v, al, be, [0, 5, 2]))


def test_commit_splits_over_the_prefix():
    # committing a prefix, then the rest of it from the new state, equals committing it at once
    rng = np.random.default_rng(3)
    S, k, v, al, be = gen.gdn_inputs(rng, 1, 8, 1, 16, 12)
    whole = gdn.commit(S, k, v, al, be, [6])
    first = gdn.commit(S, k, v, al, be, [2])
    rest = gdn.commit(first, k[:, 3:], v[:, 3:], al[:, 3:], be[:, 3:], [3])
    assert np.allclose(whole, rest, rtol=1e-13, atol=1e-13)


def test_exact_rationals_tiny_state():
    rng = np.random.default_rng(4)
    dk, dv, T = 3, 2, 3
    S = rng.integers(-3, 4, (1, 1, dv, dk)).astype(np.float64)
    k = rng.integers(-2, 3, (1, T, 1, dk)).astype(np.float64) / 4
    v = rng.integers(-5, 6, (1, T, 1, dv)).astype(np.float64) / 2
    al = np.array([0.75, 0.5, 1.0]).reshape(1, T, 1)
    be = np.array([0.25, 1.0, 0.5]).reshape(1, T, 1)
    out = gdn.commit(S, k, v, al, be, [2])[0, 0]
    M = [[Fraction(float(x)) for x in row] for row in S[0, 0]]
    for t in range(T):
        kk = [Fraction(float(x)) for x in k[0, t, 0]]
        vv = [Fraction(float(x)) for x in v[0, t, 0]]
        a, b = Fraction(float(al[0, t, 0])), Fraction(float(be[0, t, 0]))
        Sk = [sum(M[i][j] * kk[j] for j in range(dk)) for i in range(dv)]
        M = [[a * (M[i][j] - b * Sk[i] * kk[j]) + b * vv[i] * kk[j] for j in range(dk)]
             for i in range(dv)]
    assert np.array_equal(out, np.array([[float(x) for x in row] for row in M]))
