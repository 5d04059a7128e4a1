"""Pins for the oracle's int4 unpacking and group dequantisation.

The packing helpers in ``gen`` and the unpacking in ``oracle.quant`` are
written independently; hand-built words pin both to the nibble-order reading
(nibble j at bits 4j..4j+3, 8 consecutive k per weight word, 8 consecutive n
per zero-point word).
"""
import numpy as np
import pytest

import gen
from oracle import quant


def test_unpack_pack_roundtrip_exhaustive_values_and_positions():
    # every value 0..15 at every nibble position of a weight word
    q = np.zeros((8 * 16, 3), dtype=np.int64)
    for val in range(16):
        for j in range(8):
            q[8 * val + j, :] = val  # word `val` has all nibbles == val
    q[5, 1] = 3
    words = gen.pack_int4_along_k(q)
    assert np.array_equal(quant.unpack_weights(words), q)
    z = np.arange(16 * 8).reshape(16, 8) % 16
    zw = gen.pack_int4_along_n(z)
    assert np.array_equal(quant.unpack_zeros(zw), z)


def test_pack_unpack_random_words_with_top_bit():
    rng = np.random.default_rng(7)
    words = rng.integers(0, 1 << 32, size=(32, 24), dtype=np.uint32).view(np.int32)
    assert (words < 0).any()      # arithmetic-shift bugs would show on these
    assert np.array_equal(gen.pack_int4_along_k(quant.unpack_weights(words)), words)
    assert np.array_equal(gen.pack_int4_along_n(quant.unpack_zeros(words)), words)


@pytest.mark.parametrize("j", range(8))
def test_hand_built_one_hot_weight_word(j):
    # word (i=2, n=5) = 0xF << 4j, everything else zero; z = 0, s = 1
    k, n = 64, 16
    qw = np.zeros((k // 8, n), dtype=np.uint32)
    qw[2, 5] = np.uint32(0xF) << np.uint32(4 * j)
    qw = qw.view(np.int32)
    q = quant.unpack_weights(qw)
    expect = np.zeros((k, n), dtype=np.int64)
    expect[8 * 2 + j, 5] = 15
    assert np.array_equal(q, expect)


@pytest.mark.parametrize("j", range(8))
def test_hand_built_one_hot_zero_word(j):
    g, n = 3, 32
    qz = np.zeros((g, n // 8), dtype=np.uint32)
    qz[1, 2] = np.uint32(0x9) << np.uint32(4 * j)
    z = quant.unpack_zeros(qz.view(np.int32))
    expect = np.zeros((g, n), dtype=np.int64)
    expect[1, 8 * 2 + j] = 9
    assert np.array_equal(z, expect)


def test_group_to_scale_mapping_at_boundaries():
    # q - z = 1 everywhere; group g has scale 2^-g in column n (and 2^-(g+3) elsewhere);
    # the row k of W must carry the scale of group k // 128, including k = 127, 128, 255, 256.
    k, n = 512, 8
    q = np.full((k, n), 9, dtype=np.int64)
    z = np.full((k // 128, n), 8, dtype=np.int64)
    s = np.empty((k // 128, n), dtype=np.float16)
    for g in range(k // 128):
        s[g, :] = 2.0 ** -(g + 3)
        s[g, 3] = 2.0 ** -g
    w = quant.dequantize(gen.pack_int4_along_k(q), s, gen.pack_int4_along_n(z))
    for kk in (0, 127, 128, 255, 256, 383, 384, 511):
        assert w[kk, 3] == 2.0 ** -(kk // 128)
        assert w[kk, 0] == 2.0 ** -(kk // 128 + 3)


def test_dequant_signs_and_extremes():
    # q - z spans -15..15; scale 0.5 -> exact products
    q = np.array([[0], [15], [7], [8], [0], [15], [3], [12]], dtype=np.int64)
    q = np.tile(q, (16, 8))          # K = 128, N = 8
    z = np.zeros((1, 8), dtype=np.int64)
    z[0, :] = [15, 0, 7, 8, 3, 12, 1, 14]
    s = np.full((1, 8), 0.5, dtype=np.float16)
    w = quant.dequantize(gen.pack_int4_along_k(q), s, gen.pack_int4_along_n(z))
    assert np.array_equal(w, 0.5 * (q - z[[0] * 128, :]))
    assert w.min() == -7.5 and w.max() == 7.5


def test_dequantize_columns_matches_full():
    rng = np.random.default_rng(3)
    lin = gen.qlinear(rng, 256, 64)
    full = quant.dequantize(lin.qweight, lin.scales, lin.qzeros)
    cols = np.array([0, 7, 8, 33, 63])
    assert np.array_equal(quant.dequantize_columns(lin.qweight, lin.scales, lin.qzeros, cols),
                          full[:, cols])


def test_group_to_scale_mapping_at_boundaries_group_32():
    # Group size 32 (results page, section 5: team #5's compressed-tensors target):
    # row k carries the scale and zero-point of group k // 32, including k = 31, 32, 63, 64.
    k, n = 256, 8
    q = np.full((k, n), 9, dtype=np.int64)
    z = np.empty((k // 32, n), dtype=np.int64)
    s = np.empty((k // 32, n), dtype=np.float16)
    for g in range(k // 32):
        z[g, :] = 8 - (g % 3)                     # q - z = 1 + g % 3
        s[g, :] = 2.0 ** -(g + 3)
        s[g, 5] = 2.0 ** -g
    w = quant.dequantize(gen.pack_int4_along_k(q), s, gen.pack_int4_along_n(z), group_size=32)
    for kk in (0, 31, 32, 63, 64, 95, 96, 127, 128, 255):
        g = kk // 32
        assert w[kk, 5] == (1 + g % 3) * 2.0 ** -g
        assert w[kk, 0] == (1 + g % 3) * 2.0 ** -(g + 3)
    cols = np.array([0, 5, 7])
    assert np.array_equal(quant.dequantize_columns(gen.pack_int4_along_k(q), s,
                                                   gen.pack_int4_along_n(z), cols, group_size=32),
                          w[:, cols])
