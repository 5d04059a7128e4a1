"""Checks of the seeded input module: reproducibility, value distributions,
and the draft constructions' accepted-length laws."""
import math

import numpy as np
import pytest

import gen
from oracle import quant, verify


def test_seeds_reproduce_bytes_and_differ_across_seeds():
    a = gen.make_workload(1)
    b = gen.make_workload(1)
    c = gen.make_workload(1, seed_offset=1)
    assert a.x.tobytes() == b.x.tobytes()
    for la, lb in zip(a.linears, b.linears):
        assert la.qweight.tobytes() == lb.qweight.tobytes()
        assert la.scales.tobytes() == lb.scales.tobytes()
        assert la.qzeros.tobytes() == lb.qzeros.tobytes()
    assert a.lm_w.tobytes() == b.lm_w.tobytes()
    assert a.x.tobytes() != c.x.tobytes()


def test_value_distributions():
    rng = np.random.default_rng(0)
    lin = gen.qlinear(rng, 2560, 2560)
    q = quant.unpack_weights(lin.qweight)
    z = quant.unpack_zeros(lin.qzeros)
    n = q.size
    assert abs(q.mean() - 7.5) < 5 * math.sqrt(21.25 / n)
    assert abs(q.var() - 21.25) < 0.05
    assert q.min() == 0 and q.max() == 15
    assert abs(z.mean() - 7.5) < 5 * math.sqrt(21.25 / z.size)
    s = lin.scales.astype(np.float64)
    assert s.min() >= float(np.float16(0.005)) and s.max() <= float(np.float16(0.02))
    x = gen.activations(rng, 64, 2560).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.var() - 1) < 0.02
    w8 = gen.lmhead_weights(rng, 4096, 256)
    assert w8.min() == -127 and w8.max() == 127
    s8 = gen.lmhead_scales(rng, 4096).astype(np.float64)
    assert s8.min() >= float(np.float16(0.001)) and s8.max() <= float(np.float16(0.004))


def test_sigma_w_closed_form_matches_sample():
    rng = np.random.default_rng(2)
    lin = gen.qlinear(rng, 1024, 1024)
    w = quant.dequantize(lin.qweight, lin.scales, lin.qzeros)
    assert abs(w.std() / gen.SIGMA_W - 1) < 0.01


def _verify_rows(rng, cfg, t_rows):
    d, r = gen.make_drafts(rng, cfg, t_rows.reshape(-1))
    acc, _ = verify.greedy_verify(t_rows, d, cfg.vocab)
    return acc, r


@pytest.mark.parametrize("cid", [1, 3, 4])
def test_draft_construction_gives_intended_acceptance(cid):
    cfg = gen.CONFIGS[cid]
    rng = np.random.default_rng(100 + cid)
    for _ in range(200):
        t = rng.integers(0, cfg.vocab, size=(cfg.batch, cfg.k_draft + 1))
        acc, r = _verify_rows(rng, cfg, t)
        assert np.array_equal(acc, r)


def test_geometric_acceptance_mean():
    # r = min(15, G), P(G = j) = 0.75^j 0.25 (j >= 0): E[r] = sum_{k=1}^{15} 0.75^k
    p_ge = [0.75 ** k for k in range(1, 16)]
    mean = sum(p_ge)
    second = sum((2 * k - 1) * 0.75 ** k for k in range(1, 16))
    var = second - mean ** 2
    assert abs(mean + 1 - 3.960) < 5e-4
    rng = np.random.default_rng(5)
    n = 20000
    rs = np.array([gen.draw_r_geometric(rng, 15) for _ in range(n)])
    assert abs(rs.mean() - mean) < 3 * math.sqrt(var / n)
    assert rs.max() == 15 and rs.min() == 0


def test_padded_acceptance_mean():
    # L ~ U{0..20}, r | L ~ U{0..L}: E[r] = 5, Var(r) = 200/9
    rng = np.random.default_rng(6)
    n = 20000
    t = np.arange(21)
    rs = []
    n_sent = 0
    for _ in range(n):
        d, r = gen.padded_drafts(rng, t, 20, 151936)
        rs.append(r)
        n_sent += int((d == -1).sum())
    rs = np.array(rs)
    assert abs(rs.mean() - 5.0) < 3 * math.sqrt((200 / 9) / n)
    assert abs(n_sent / n - 10.0) < 0.2            # E[20 - L] = 10 sentinels


def test_uniform_acceptance_mean():
    rng = np.random.default_rng(7)
    n = 20000
    rs = np.array([gen.draw_r_uniform(rng, 15) for _ in range(n)])
    assert abs(rs.mean() - 7.5) < 3 * math.sqrt((16 ** 2 - 1) / 12 / n)


def test_chain_alpha_keeps_unit_rms():
    rng = np.random.default_rng(8)
    lin = gen.qlinear(rng, 2560, 512)
    x = gen.activations(rng, 16, 2560)
    w = quant.dequantize(lin.qweight, lin.scales, lin.qzeros)
    y = gen.chain_alpha(2560) * (x.astype(np.float64) @ w)
    assert 0.9 < y.std() < 1.1


def test_config_shapes():
    plan3 = gen.chain_plan(gen.CONFIGS[3])
    assert len(plan3) == 144
    assert [p[:2] for p in plan3[:4]] == [(2560, 6144), (4096, 2560), (2560, 19456), (9728, 2560)]
    # 36 layers of weights, scales and zero-points: ~1.9 GB
    per_layer = sum(k * n // 2 + (k // 128) * n * 2 + (k // 128) * n // 2 for k, n, _ in plan3[:4])
    assert per_layer * 36 == 1_887_621_120
    assert gen.chain_plan(gen.CONFIGS[5]) == [(2560, 19456, 1.0), (9728, 2560, 1.0)]


def test_drafter_reading_matches_page_size():
    """The 4-bit drafter reading (fusion of five 2560-wide taps, then five layers of the
    target's linears) holds 279.2 MB of weights, scales and zeros: within 1% of the
    277 MB the results page gives for team #3's W4A16 g128 drafter (section 5)."""
    lins = gen.drafter_linears()
    assert len(lins) == 1 + 4 * gen.DRAFTER_LAYERS
    assert (lins[0].k_in, lins[0].n_out) == (5 * gen.HIDDEN, gen.HIDDEN)
    total = sum(l.k_in * l.n_out // 2 + (l.k_in // 128) * l.n_out * 2
                + (l.k_in // 128) * (l.n_out // 8) * 4 for l in lins)
    assert total == 279_193_600
    assert abs(total / 277e6 - 1) < 0.01
    # each linear reads the leading columns of the previous output
    for prev, cur in zip(lins, lins[1:]):
        assert cur.k_in <= prev.n_out


def test_drafter_workload_is_seeded():
    a = gen.make_drafter_workload()
    b = gen.make_drafter_workload()
    assert a.x.shape == (16, 5 * gen.HIDDEN) and a.x.dtype == np.float16
    assert a.x.tobytes() == b.x.tobytes()
    assert all(la.qweight.tobytes() == lb.qweight.tobytes() for la, lb in zip(a.linears, b.linears))
    assert [p[:2] for p in gen.drafter_plan()] == [(l.k_in, l.n_out) for l in gen.drafter_linears()]
