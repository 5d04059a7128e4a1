"""Pins for the oracle's 8-bit lm_head, argmax tie-break and top-2 margin."""
from fractions import Fraction

import numpy as np

import gen
from oracle import lmhead


def test_one_hot_hidden_reads_one_weight_column():
    rng = np.random.default_rng(21)
    v, h = 50, 64
    w8 = gen.lmhead_weights(rng, v, h)
    s8 = gen.lmhead_scales(rng, v)
    hid = np.zeros((2, h), dtype=np.float16)
    hid[0, 10] = 1.0
    hid[1, 63] = 1.0
    lg = lmhead.logits(hid, w8, s8)
    assert np.array_equal(lg[0], s8.astype(np.float64) * w8[:, 10])
    assert np.array_equal(lg[1], s8.astype(np.float64) * w8[:, 63])
    t, top, _ = lmhead.argmax_margin(lg)
    expect = s8.astype(np.float64) * w8[:, 10]
    assert t[0] == int(np.flatnonzero(expect == expect.max())[0])


def test_planted_winner_and_margin():
    rng = np.random.default_rng(23)
    v, h = 300, 128
    w8 = gen.lmhead_weights(rng, v, h)
    s8 = np.full(v, 0.002, dtype=np.float16)
    hid = gen.activations(rng, 1, h)
    sign = np.where(hid[0] >= 0, 127, -127).astype(np.int8)
    w8[123] = sign                       # maximises the dot product over int8 rows
    t, top, margin = lmhead.lmhead_argmax(hid, w8, s8)
    assert t[0] == 123
    assert margin[0] > 0
    lg = lmhead.logits(hid, w8, s8)[0]
    assert top[0] == lg[123]
    assert margin[0] == lg[123] - np.max(np.delete(lg, 123))


def test_exact_tie_goes_to_lowest_index_with_zero_margin():
    rng = np.random.default_rng(29)
    v, h = 40, 32
    w8 = gen.lmhead_weights(rng, v, h)
    s8 = np.full(v, 0.003, dtype=np.float16)
    hid = gen.activations(rng, 1, h)
    best = np.where(hid[0] >= 0, 127, -127).astype(np.int8)
    w8[31] = best
    w8[9] = best
    t, _, margin = lmhead.lmhead_argmax(hid, w8, s8)
    assert t[0] == 9
    assert margin[0] == 0.0


def test_int8_minus_128_is_handled():
    w8 = np.array([[-128, 0], [127, 0]], dtype=np.int8)
    s8 = np.array([1.0, 1.0], dtype=np.float16)
    hid = np.array([[-1.0, 0.0]], dtype=np.float16)
    lg = lmhead.logits(hid, w8, s8)
    assert lg[0, 0] == 128.0 and lg[0, 1] == -127.0


def test_brute_force_exact_rationals():
    rng = np.random.default_rng(31)
    v, h, m = 7, 32, 3
    w8 = gen.lmhead_weights(rng, v, h)
    s8 = gen.lmhead_scales(rng, v)
    hid = gen.activations(rng, m, h)
    lg = lmhead.logits(hid, w8, s8)
    for mm in range(m):
        exact = []
        for vv in range(v):
            acc = sum(Fraction(float(hid[mm, kk])) * int(w8[vv, kk]) for kk in range(h))
            exact.append(Fraction(float(s8[vv])) * acc)
        for vv in range(v):
            assert abs(lg[mm, vv] - float(exact[vv])) <= 1e-13 * max(1.0, abs(float(exact[vv])))
        best = max(exact)
        t_exact = min(i for i, e in enumerate(exact) if e == best)
        t, _, _ = lmhead.argmax_margin(lg[mm:mm + 1])
        assert t[0] == t_exact


def test_chunking_boundary_is_seamless():
    rng = np.random.default_rng(37)
    v, h = lmhead._CHUNK + 5, 16
    w8 = gen.lmhead_weights(rng, v, h)
    s8 = gen.lmhead_scales(rng, v)
    hid = gen.activations(rng, 2, h)
    lg = lmhead.logits(hid, w8, s8)
    for vv in (0, lmhead._CHUNK - 1, lmhead._CHUNK, v - 1):
        direct = (hid.astype(np.float64) @ w8[vv].astype(np.float64)) * float(s8[vv])
        assert np.allclose(lg[:, vv], direct, rtol=1e-15, atol=0)


def test_f16_one_hot_hidden_and_brute_force():
    rng = np.random.default_rng(41)
    v, h = 30, 40
    w = gen.f16_weights(rng, v, h)
    hid = np.zeros((2, h), dtype=np.float16)
    hid[0, 7] = 1.0
    hid[1, 39] = -2.0
    lg = lmhead.logits_f16(hid, w)
    assert np.array_equal(lg[0], w[:, 7].astype(np.float64))
    assert np.array_equal(lg[1], -2.0 * w[:, 39].astype(np.float64))
    x = gen.activations(rng, 2, h)
    lg = lmhead.logits_f16(x, w)
    for mm in range(2):
        for vv in range(v):
            exact = sum(Fraction(float(x[mm, kk])) * Fraction(float(w[vv, kk])) for kk in range(h))
            assert abs(lg[mm, vv] - float(exact)) <= 1e-13 * max(1.0, abs(float(exact)))


def test_f16_planted_winner_across_the_chunk_seam():
    # rows on both sides of the 8192-row slice boundary; the winner sits right after it
    rng = np.random.default_rng(43)
    v, h = 8192 + 100, 16
    w = np.zeros((v, h), dtype=np.float16)
    w[8191, 3] = np.float16(0.5)
    w[8192, 3] = np.float16(0.625)
    hid = np.zeros((1, h), dtype=np.float16)
    hid[0, 3] = 2.0
    t, top, margin = lmhead.lmhead_argmax_f16(hid, w)
    assert t[0] == 8192 and top[0] == 1.25 and margin[0] == 0.25
