"""GPU parity of the 8-bit lm_head with fused argmax (G2), greedy verify (G4)
and the fused lm_head + verify launch."""
import json
import os

import numpy as np
import pytest

import gen
from oracle import lmhead as olm, verify as over
from tests.gpu_util import MARGIN, check_argmax, dev, host, log

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "verify_cases.json")


def sync():
    import torch
    torch.cuda.synchronize()


def run_lm(w4v, h, w8, s8, ws=None):
    t, mx = w4v.w8a16_lmhead_argmax(dev(h), dev(w8), dev(s8), workspace=ws)
    sync()
    return host(t), host(mx)


@pytest.mark.parametrize("m,v", [(16, 4096), (1, 4096), (21, 1000), (16, 4097), (40, 777),
                                 (168, 5000), (16, 70000), (3, 1),
                                 (64, 3000), (65, 4099), (97, 2000), (200, 777)])
def test_random(lib, m, v):
    log(f"lmhead m={m} v={v}")
    rng = np.random.default_rng(m * 31 + v)
    w8 = gen.lmhead_weights(rng, v, gen.HIDDEN)
    s8 = gen.lmhead_scales(rng, v)
    h = gen.activations(rng, m, gen.HIDDEN)
    t, mx = run_lm(lib, h, w8, s8)
    lg = olm.logits(h, w8, s8)
    low, t_o, top, _ = check_argmax(t, lg, f"m={m} v={v}")
    sure = np.flatnonzero(t == t_o)
    assert np.allclose(mx[sure], top[sure], rtol=1e-5, atol=1e-4)
    log(f"  low-margin rows {low}/{m}")


# Blocks of at most 16 rows stage the whole hidden rows in LDS when H <= 2560 (the
# swizzled tile, fewer 128-k segments than the tile holds at small H); wider rows take
# the per-step hidden tile.  Both sides of that switch, one row and sixteen.
@pytest.mark.parametrize("m,h,v", [(16, 128, 700), (1, 1024, 3000), (16, 2432, 2100),
                                   (16, 2688, 3000), (1, 4096, 1500), (12, 5120, 900)])
def test_hidden_widths(lib, m, h, v):
    log(f"lmhead m={m} h={h} v={v}")
    rng = np.random.default_rng(7 * m + h + v)
    w8 = gen.lmhead_weights(rng, v, h)
    s8 = gen.lmhead_scales(rng, v)
    x = gen.activations(rng, m, h)
    t, mx = run_lm(lib, x, w8, s8)
    lg = olm.logits(x, w8, s8)
    low, t_o, top, _ = check_argmax(t, lg, f"m={m} h={h} v={v}")
    sure = np.flatnonzero(t == t_o)
    assert np.allclose(mx[sure], top[sure], rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("m", [16, 100])
def test_ties_go_to_lowest_index(lib, m):
    rng = np.random.default_rng(5 + m)
    v = 25000
    w8 = gen.lmhead_weights(rng, v, gen.HIDDEN)
    s8 = np.full(v, 0.002, dtype=np.float16)
    h = gen.activations(rng, m, gen.HIDDEN)
    win = np.where(h >= 0, 127, -127).astype(np.int8)      # the largest int8 dot product for row i
    cands = {i: (12000 + 31 * i, 500 + 7 * i, 19000 + 50 * i) for i in range(m)}   # disjoint
    for i in range(m):
        for idx in cands[i]:
            w8[idx] = win[i]
    t, _ = run_lm(lib, h, w8, s8)
    t_o, _, margin = olm.argmax_margin(olm.logits(h, w8, s8))
    for i in range(m):
        assert margin[i] == 0.0                 # an exact three-way tie
        assert t_o[i] == min(cands[i])
        assert t[i] == min(cands[i])


@pytest.mark.parametrize("m", [16, 168])
def test_int8_extremes(lib, m):
    rng = np.random.default_rng(6 + m)
    v = 3000
    w8 = rng.choice(np.array([-128, -127, 127], dtype=np.int8), size=(v, gen.HIDDEN))
    s8 = gen.lmhead_scales(rng, v)
    h = gen.activations(rng, m, gen.HIDDEN)
    t, _ = run_lm(lib, h, w8, s8)
    check_argmax(t, olm.logits(h, w8, s8), "extremes")


@pytest.mark.parametrize("m", [16, 168])
def test_one_hot_hidden(lib, m):
    rng = np.random.default_rng(8 + m)
    v = 5000
    w8 = gen.lmhead_weights(rng, v, gen.HIDDEN)
    s8 = gen.lmhead_scales(rng, v)
    h = np.zeros((m, gen.HIDDEN), dtype=np.float16)
    for i in range(m):
        h[i, (157 * i + 3) % gen.HIDDEN] = 1.0
    t, mx = run_lm(lib, h, w8, s8)
    lg = olm.logits(h, w8, s8)
    t_o, top, _ = olm.argmax_margin(lg)
    assert np.array_equal(t, t_o)           # logits are exact products: ties broken identically
    assert np.array_equal(mx, top.astype(np.float32))


@pytest.mark.parametrize("m", [16, 168])
def test_full_vocabulary(lib, m):
    rng = np.random.default_rng(m)
    r_lm = np.random.default_rng(2024)
    w8 = gen.lmhead_weights(r_lm, gen.VOCAB, gen.HIDDEN)
    s8 = gen.lmhead_scales(r_lm, gen.VOCAB)
    h = gen.activations(rng, m, gen.HIDDEN)
    log(f"lmhead full vocab m={m}")
    need = lib.lmhead_workspace_size(m, gen.HIDDEN, gen.VOCAB)
    ws = lib.new_workspace(need)
    t1, _ = run_lm(lib, h, w8, s8, ws)
    t2, _ = run_lm(lib, h, w8, s8, ws)       # workspace reused: same answer
    assert np.array_equal(t1, t2)
    low, *_ = check_argmax(t1, olm.logits(h, w8, s8), f"full vocab m={m}")
    log(f"  low-margin rows {low}/{m}")


# ------------------------------------------------------------------ greedy verify (G4)
def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_verify_golden(lib, case):
    k = len(case["drafts"])
    t = np.array([case["target"]], dtype=np.int32)
    d = np.array(case["drafts"], dtype=np.int32).reshape(1, k)
    acc, out = lib.greedy_verify(dev(t), dev(d), case["vocab"])
    sync()
    assert int(host(acc)[0]) == case["accepted_len"]
    assert host(out)[0].tolist() == case["out_tokens"]


@pytest.mark.parametrize("b,k", [(1, 15), (8, 20), (300, 7), (5, 0), (1000, 1)])
def test_verify_random_batches(lib, b, k):
    v = 50
    rng = np.random.default_rng(b * 100 + k)
    t = rng.integers(0, v, size=(b, k + 1)).astype(np.int32)
    d = np.empty((b, k), dtype=np.int32)
    for i in range(b):
        r = rng.integers(0, k + 1)
        d[i] = rng.integers(-1, v + 3, size=k)        # sentinels and out-of-range ids too
        d[i, :r] = t[i, :r]
    acc, out = lib.greedy_verify(dev(t), dev(d), v)
    sync()
    a_o, out_o = over.greedy_verify(t, d, v)
    assert np.array_equal(host(acc), a_o)
    assert np.array_equal(host(out), out_o)


@pytest.mark.parametrize("b,k,v", [(1, 15, 4096), (8, 20, 30000), (2, 0, 500)])
def test_fused_lmhead_verify(lib, b, k, v):
    rng = np.random.default_rng(b + k + v)
    w8 = gen.lmhead_weights(rng, v, gen.HIDDEN)
    s8 = gen.lmhead_scales(rng, v)
    m = b * (k + 1)
    h = gen.activations(rng, m, gen.HIDDEN)
    t_o, _, margin = olm.lmhead_argmax(h, w8, s8)
    cfg = gen.Config(0, "t", m=m, layers=0, vocab=v, batch=b, k_draft=k,
                     draft_mode="padded" if k else "uniform_r")
    if k:
        drafts, r = gen.make_drafts(rng, cfg, t_o)
    else:
        drafts = np.zeros((b, 0), dtype=np.int32)
    t_g, mx, acc, out = lib.w8a16_lmhead_argmax_verify(dev(h), dev(w8), dev(s8), dev(drafts))
    sync()
    t_g = host(t_g)
    sure = margin > MARGIN
    assert np.array_equal(t_g[sure], t_o[sure])
    # the fused scan must agree exactly with the oracle scan on the GPU's ids
    a_o, out_o = over.greedy_verify(t_g.reshape(b, k + 1), drafts, v)
    assert np.array_equal(host(acc), a_o)
    assert np.array_equal(host(out), out_o)
    # and with the separate verify kernel
    acc2, out2 = lib.greedy_verify(dev(t_g.reshape(b, k + 1).astype(np.int32)), dev(drafts), v)
    sync()
    assert np.array_equal(host(acc2), a_o) and np.array_equal(host(out2), out_o)
