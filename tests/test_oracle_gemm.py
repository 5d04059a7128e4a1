"""Pins for the oracle's W4A16 linear: identity and one-hot weights, closed
forms, and an exact-rational brute force on a tiny shape."""
from fractions import Fraction

import numpy as np
import pytest

import gen
from oracle import gemm, quant


def _identity_encodings(n):
    """Three encodings of W = I (K = N): returns list of (q, z, s)."""
    eye = np.eye(n, dtype=np.int64)
    g = n // 128
    out = []
    out.append((eye.copy(), np.zeros((g, n), np.int64), np.ones((g, n), np.float16)))
    out.append((8 + eye, np.full((g, n), 8, np.int64), np.ones((g, n), np.float16)))
    out.append((7 + 2 * eye, np.full((g, n), 7, np.int64), np.full((g, n), 0.5, np.float16)))
    return out


@pytest.mark.parametrize("enc", range(3))
def test_identity_weights_reproduce_x_bit_exactly(enc):
    n = 256
    q, z, s = _identity_encodings(n)[enc]
    rng = np.random.default_rng(11)
    x = gen.activations(rng, 5, n)
    y = gemm.w4a16_gemm(x, gen.pack_int4_along_k(q), s, gen.pack_int4_along_n(z))
    assert np.array_equal(gemm.to_fp16(y), x)


def test_one_hot_weight_selects_one_input_column():
    k, n = 384, 24
    k0, n0 = 200, 17                   # k0 in group 1
    q = np.full((k, n), 5, dtype=np.int64)
    z = np.full((k // 128, n), 5, dtype=np.int64)
    q[k0, n0] = 9                      # q - z = 4, scale 0.25 -> w = 1
    s = np.full((k // 128, n), 0.25, dtype=np.float16)
    rng = np.random.default_rng(5)
    x = gen.activations(rng, 3, k)
    y = gemm.w4a16_gemm(x, gen.pack_int4_along_k(q), s, gen.pack_int4_along_n(z))
    expect = np.zeros((3, n))
    expect[:, n0] = x[:, k0].astype(np.float64)
    assert np.array_equal(y, expect)


def test_q_equal_z_gives_zero():
    rng = np.random.default_rng(9)
    k, n = 256, 16
    z = rng.integers(0, 16, size=(k // 128, n))
    q = np.repeat(z, 128, axis=0)
    s = gen.group_scales(rng, k // 128, n)
    x = gen.activations(rng, 4, k)
    y = gemm.w4a16_gemm(x, gen.pack_int4_along_k(q), s, gen.pack_int4_along_n(z), alpha=3.0)
    assert not np.any(y)


def test_constant_dequant_gives_scaled_row_sums():
    rng = np.random.default_rng(13)
    k, n, c = 384, 8, -3
    z = np.full((k // 128, n), 10, dtype=np.int64)
    q = np.full((k, n), 10 + c, dtype=np.int64)
    s = np.full((k // 128, n), 0.0078125, dtype=np.float16)   # 2^-7
    x = gen.activations(rng, 6, k)
    alpha = 0.5
    y = gemm.w4a16_gemm(x, gen.pack_int4_along_k(q), s, gen.pack_int4_along_n(z), alpha=alpha)
    rowsum = x.astype(np.float64).sum(axis=1)
    assert np.allclose(y, (alpha * 0.0078125 * c * rowsum)[:, None], rtol=1e-14, atol=1e-14)


def test_brute_force_exact_rationals_tiny_shape():
    rng = np.random.default_rng(17)
    m, k, n = 2, 256, 16
    lin = gen.qlinear(rng, k, n)
    x = gen.activations(rng, m, k)
    alpha = 0.75
    y = gemm.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros, alpha=alpha)
    # exact rationals from the raw words, independent of numpy's unpacking
    words = lin.qweight.view(np.uint32)
    zwords = lin.qzeros.view(np.uint32)
    for mm in range(m):
        for nn in range(n):
            acc = Fraction(0)
            for kk in range(k):
                qv = (int(words[kk // 8, nn]) >> (4 * (kk % 8))) & 15
                zv = (int(zwords[kk // 128, nn // 8]) >> (4 * (nn % 8))) & 15
                sv = Fraction(float(lin.scales[kk // 128, nn]))
                acc += Fraction(float(x[mm, kk])) * sv * (qv - zv)
            exact = Fraction(alpha) * acc
            assert abs(y[mm, nn] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def test_columns_variant_matches_full_product():
    rng = np.random.default_rng(19)
    lin = gen.qlinear(rng, 256, 48)
    x = gen.activations(rng, 3, 256)
    cols = np.array([1, 8, 40, 47])
    full = gemm.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros, alpha=2.0)
    part = gemm.w4a16_gemm_columns(x, lin.qweight, lin.scales, lin.qzeros, cols, alpha=2.0)
    assert np.allclose(part, full[:, cols], rtol=1e-15, atol=0)


def test_fp16_storage_rounds_to_nearest_even():
    vals = np.array([1.0 + 2.0 ** -11,                 # tie -> even (1.0)
                     1.0 + 3 * 2.0 ** -11,             # tie -> even (1 + 2^-9)
                     1.0 + 2.0 ** -11 + 2.0 ** -40,    # just above the tie -> up
                     -(1.0 + 2.0 ** -11 + 2.0 ** -40),
                     65504.0, 65520.0,                 # max finite, first that overflows
                     2.0 ** -25, 2.0 ** -25 + 2.0 ** -40])   # subnormal tie and just above
    got = gemm.to_fp16(vals)
    assert got[0] == np.float16(1.0)
    assert got[1] == np.float16(1.0 + 2.0 ** -9)
    assert got[2] == np.float16(1.0 + 2.0 ** -10)
    assert got[3] == np.float16(-(1.0 + 2.0 ** -10))
    assert got[4] == np.float16(65504.0)
    assert np.isinf(got[5])
    assert got[6] == 0.0
    assert got[7] == np.float16(2.0 ** -24)


def test_brute_force_exact_rationals_group_32():
    rng = np.random.default_rng(23)
    m, k, n = 2, 128, 16
    lin = gen.qlinear(rng, k, n, group_size=32)
    assert lin.scales.shape == (4, n) and lin.qzeros.shape == (4, n // 8)
    x = gen.activations(rng, m, k)
    y = gemm.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros, alpha=1.25, group_size=32)
    words = lin.qweight.view(np.uint32)
    zwords = lin.qzeros.view(np.uint32)
    for mm in range(m):
        for nn in range(n):
            acc = Fraction(0)
            for kk in range(k):
                qv = (int(words[kk // 8, nn]) >> (4 * (kk % 8))) & 15
                zv = (int(zwords[kk // 32, nn // 8]) >> (4 * (nn % 8))) & 15
                sv = Fraction(float(lin.scales[kk // 32, nn]))
                acc += Fraction(float(x[mm, kk])) * sv * (qv - zv)
            exact = Fraction(1.25) * acc
            assert abs(y[mm, nn] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def test_f16_linear_identity_and_one_hot():
    rng = np.random.default_rng(29)
    x = gen.activations(rng, 3, 64)
    eye = np.eye(64, dtype=np.float16)
    assert np.array_equal(gemm.to_fp16(gemm.f16_linear(x, eye)).view(np.uint16), x.view(np.uint16))
    w = np.zeros((40, 64), dtype=np.float16)
    w[17, 9] = np.float16(0.375)                       # output 17 reads input 9
    y = gemm.f16_linear(x, w, alpha=2.0)
    expect = np.zeros((3, 40))
    expect[:, 17] = 0.75 * x[:, 9].astype(np.float64)
    assert np.array_equal(y, expect)


def test_f16_linear_brute_force_exact_rationals():
    rng = np.random.default_rng(31)
    m, k, n = 2, 48, 5
    x = gen.activations(rng, m, k)
    w = gen.f16_weights(rng, n, k)
    y = gemm.f16_linear(x, w, alpha=0.5)
    for mm in range(m):
        for nn in range(n):
            exact = Fraction(1, 2) * sum(Fraction(float(x[mm, kk])) * Fraction(float(w[nn, kk]))
                                         for kk in range(k))
            assert abs(y[mm, nn] - float(exact)) <= 1e-13 * max(1.0, abs(float(exact)))
    assert w.dtype == np.float16 and w.shape == (n, k)
