"""GPU parity of the half-precision parts of team #5's target (results page,
section 5: first two and last two layers and the lm_head kept in fp16) against
the fp64 oracle: the fp16 linear (vendor library GEMM) at the 4B-class shapes,
strided operands and graph replay; the fp16 lm_head with fused argmax (G2)
and greedy verify (G4 on the GPU's own target ids, G3 free-running)."""
import numpy as np
import pytest

import gen
from oracle import gemm as og, lmhead as olm, verify as over
from tests.gpu_util import MARGIN, check_argmax, check_gemm, dev, host, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m,k,n", [
    (16, 2560, 6144), (16, 4096, 2560), (16, 2560, 19456), (16, 9728, 2560),
    (24, 2560, 6144), (24, 9728, 2560),          # the verify block of K = 23
    (1, 2560, 520), (5, 384, 136), (21, 1280, 1032), (32, 128, 8),
    (16, 200, 136), (24, 1000, 520),             # K not a multiple of 128
    (33, 1280, 1032), (640, 1280, 1032),
])
def test_f16_linear_shapes(lib, m, k, n):
    import torch
    rng = np.random.default_rng(7000 + m + k + n)
    w = gen.f16_weights(rng, n, k)
    x = gen.activations(rng, m, k)
    y = lib.f16_gemm(dev(x), dev(w), alpha=0.5)
    torch.cuda.synchronize()
    rel, mx = check_gemm(host(y), og.f16_linear(x, w, alpha=0.5), f"f16 {m}x{k}x{n}")
    log(f"  f16 {m}x{k}x{n}: rel-L2 {rel:.2e}")


def test_f16_linear_strided_and_graph_replay(lib):
    """x and w as column slices of wider tensors, y a strided view; a captured call replays
    bit-identically to the eager one, with eager work between the replays."""
    import torch
    rng = np.random.default_rng(71)
    m, k, n = 16, 2560, 2560
    xw = gen.activations(rng, m, 4096)
    ww = gen.f16_weights(rng, n, 3072)
    x_d, w_d = dev(xw)[:, :k], dev(ww)[:, :k]
    out_wide = torch.full((m, 3000), 7.0, dtype=torch.float16, device="cuda")
    y = out_wide[:, 200:200 + n]
    ws = lib.new_workspace(lib.f16_gemm_workspace_size(m, n, k))
    lib.f16_gemm(x_d, w_d, out=y, workspace=ws)
    torch.cuda.synchronize()
    full = host(out_wide)
    check_gemm(full[:, 200:200 + n], og.f16_linear(xw[:, :k], ww[:, :k]), "f16 strided")
    assert np.all(full[:, :200] == 7.0) and np.all(full[:, 200 + n:] == 7.0)
    eager = full[:, 200:200 + n].copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.f16_gemm(x_d, w_d, out=y, workspace=ws)
    for rep in range(3):
        y.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y).view(np.uint16), eager.view(np.uint16)), rep


@pytest.mark.parametrize("m,v", [(16, 4096), (16, 151936), (21, 50000), (1, 300),
                                 (64, 3000), (100, 4099), (168, 20000)])   # 64- and 96-row blocks
def test_f16_lmhead_argmax(lib, m, v):
    import torch
    rng = np.random.default_rng(8000 + m + v)
    hdim = 2560
    w = gen.f16_weights(rng, v, hdim)
    h = gen.activations(rng, m, hdim)
    ids, mx, _, _ = lib.f16_lmhead_argmax_verify(dev(h), dev(w))
    torch.cuda.synchronize()
    lg = olm.logits_f16(h, w)
    low, t, top, margin = check_argmax(host(ids), lg, f"f16 lm_head m={m} v={v}")
    sure = margin > MARGIN
    assert np.allclose(host(mx)[sure], top[sure], rtol=1e-4, atol=1e-4)
    log(f"  f16 lm_head m={m} v={v}: {low} low-margin rows")


def test_f16_lmhead_exact_tie_goes_to_lowest_index(lib):
    import torch
    v, hdim = 9000, 256
    w = np.zeros((v, hdim), dtype=np.float16)
    for r in (17, 4321, 8999):                      # three rows share the maximum
        w[r, :] = np.float16(0.25)
    w[100, :] = np.float16(0.125)
    h = np.ones((16, hdim), dtype=np.float16)
    ids, mx, _, _ = lib.f16_lmhead_argmax_verify(dev(h), dev(w))
    torch.cuda.synchronize()
    assert np.all(host(ids) == 17)
    assert np.all(host(mx) == 64.0)


def test_f16_lmhead_fused_verify(lib):
    """Drafts built from the oracle's own target ids with planted accepted lengths; the fused
    verify must match the oracle's acceptance on the GPU's ids (G4) and the planted lengths
    wherever every consulted row is clear (G3)."""
    import torch
    rng = np.random.default_rng(91)
    b, k, hdim, v = 4, 15, 2560, 151936
    w = gen.f16_weights(rng, v, hdim)
    h = gen.activations(rng, b * (k + 1), hdim)
    t_ref, _, margin = olm.lmhead_argmax_f16(h, w)
    tt = t_ref.reshape(b, k + 1)
    planted = np.array([0, 5, 15, 9])
    drafts = np.stack([gen.drafts_with_prefix(rng, tt[i], k, v, int(planted[i])) for i in range(b)])
    ids, _, acc, out = lib.f16_lmhead_argmax_verify(dev(h), dev(w), draft_ids=dev(drafts.astype(np.int32)))
    torch.cuda.synchronize()
    ids_h, acc_h, out_h = host(ids), host(acc), host(out)
    acc_g, out_g = over.greedy_verify(ids_h.reshape(b, k + 1), drafts, v)
    assert np.array_equal(acc_h, acc_g.astype(np.int32)) and np.array_equal(out_h, out_g)
    for i in range(b):
        if np.all(margin.reshape(b, k + 1)[i, :planted[i] + 1] > MARGIN):
            assert acc_h[i] == planted[i], (i, acc_h[i], planted[i])


def test_f16_linear_shares_a_workspace_with_split_k_calls(lib):
    """A workspace sized for both kinds of linear: split-K W4A16 calls before and after an
    fp16 call stay correct and the arrival counters stay at zero."""
    import torch
    rng = np.random.default_rng(73)
    k, n = 9728, 2560
    lin = gen.qlinear(rng, k, n, group_size=32)
    w16 = gen.f16_weights(rng, 2560, 2560)
    x = gen.activations(rng, 16, k)
    ws = lib.new_workspace(max(lib.gemm_workspace_size(16, n, k, 32),
                               lib.f16_gemm_workspace_size(16, 2560, 2560)))
    ref = og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros, group_size=32)
    for rep in range(2):
        y = lib.w4a16_gemm(dev(x), dev(lin.qweight), dev(lin.scales), dev(lin.qzeros),
                           workspace=ws, group_size=32)
        torch.cuda.synchronize()
        check_gemm(host(y), ref, f"split-K around fp16 call, pass {rep}")
        z = lib.f16_gemm(y, dev(w16), workspace=ws)
        torch.cuda.synchronize()
        check_gemm(host(z), og.f16_linear(host(y), w16), f"fp16 on the shared workspace, pass {rep}")
        assert int(torch.count_nonzero(ws[:65536])) == 0
