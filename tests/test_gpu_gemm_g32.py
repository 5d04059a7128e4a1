"""GPU parity of the W4A16 linear at group size 32 (results page, section 5:
team #5's compressed-tensors target) against the fp64 oracle on both paths
(M <= 32 skinny; M >= 33 the LDS-tiled MFMA kernel, split or unsplit),
exact identity and one-hot cases whose scale and zero-point change every 32 k,
and the 4B-class layer's linears at M = 16."""
import numpy as np
import pytest

import gen
from oracle import gemm as og
from tests.gpu_util import check_gemm, dev, host, log

pytestmark = pytest.mark.gpu
GS = 32


def run_gemm(w4v, x, lin, alpha=1.0, ws=None, no_ws=False):
    import torch
    y = w4v.w4a16_gemm(dev(x), dev(lin.qweight), dev(lin.scales), dev(lin.qzeros), alpha=alpha,
                       workspace=ws, group_size=GS, no_workspace=no_ws)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("m,k,n", [
    (16, 2560, 2560),          # skinny, M = 16
    (1, 2560, 520),            # one row, ragged N
    (21, 1280, 520),           # K = 20 verify block: two m-tiles
    (16, 9728, 2560),          # deep K: split across blocks
    (5, 128, 8),               # one 128-k step, four groups, narrowest N
    (33, 256, 200),            # the M >= 33 kernel, ragged rows and columns
    (200, 1280, 1032),
    (150, 1280, 520),          # 192-row block tiles
    (512, 384, 136),
    (640, 1280, 1032),
])
def test_random_shapes_group_32(lib, m, k, n):
    no_ws = lib.gemm_workspace_size(m, n, k, GS) == 0
    log(f"gemm g32 m={m} k={k} n={n} no_ws={no_ws}")
    rng = np.random.default_rng(5000 + m + k + n)
    lin = gen.qlinear(rng, k, n, group_size=GS)
    x = gen.activations(rng, m, k)
    y = run_gemm(lib, x, lin, alpha=0.75, no_ws=no_ws)
    rel, mx = check_gemm(y, og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros, alpha=0.75,
                                          group_size=GS), f"g32 {m}x{k}x{n}")
    log(f"  rel-L2 {rel:.2e} max/rms {mx:.2e}")


@pytest.mark.parametrize("enc", range(3))
@pytest.mark.parametrize("m", [1, 16, 21, 64, 200, 640])
def test_identity_weights_bit_exact_group_32(lib, enc, m):
    """q - z in {0, 1} (or {0, 2} at scale 0.5) with the zero-point changing every 32 k."""
    n = 512
    g = n // GS
    eye = np.eye(n, dtype=np.int64)
    zg = np.array([(3 * i) % 14 for i in range(g)], np.int64)       # per-group zero-points
    zrows = np.repeat(zg, GS)[:, None]                                # zero of row k's group
    q, z, s = [
        (eye, np.zeros((g, n), np.int64), np.ones((g, n), np.float16)),
        (zrows + eye, np.repeat(zg[:, None], n, 1), np.ones((g, n), np.float16)),
        (zrows + 2 * eye, np.repeat(zg[:, None], n, 1), np.full((g, n), 0.5, np.float16)),
    ][enc]
    lin = gen.QLinear(gen.pack_int4_along_k(q), s, gen.pack_int4_along_n(z), n, n, GS)
    x = gen.activations(np.random.default_rng(enc + m), m, n)
    y = run_gemm(lib, x, lin)
    assert np.array_equal(y.view(np.uint16), x.view(np.uint16))


@pytest.mark.parametrize("m", [16, 64, 300])
def test_one_hot_weight_with_per_group_scales(lib, m):
    """A single nonzero weight in the third 32-k group of a 128-k step; every group has
    its own scale and zero-point, so a group index off by one changes the result."""
    k, n = 512, 264
    k0, n0 = 128 + 2 * 32 + 5, 203                  # group 6
    g = k // GS
    zg = np.array([(5 * i + 1) % 16 for i in range(g)], np.int64)
    q = np.repeat(zg, GS)[:, None] * np.ones((1, n), np.int64)   # q = z: all weights zero
    q[k0, n0] = zg[k0 // GS] + 3 if zg[k0 // GS] <= 12 else zg[k0 // GS] - 3
    s = np.array([2.0 ** -(i % 5) for i in range(g)], np.float16)[:, None] * np.ones((1, n), np.float16)
    z = np.repeat(zg[:, None], n, 1)
    lin = gen.QLinear(gen.pack_int4_along_k(q), s.astype(np.float16), gen.pack_int4_along_n(z), k, n, GS)
    x = gen.activations(np.random.default_rng(9 + m), m, k)
    y = run_gemm(lib, x, lin)
    w = float(s[k0 // GS, n0]) * float(q[k0, n0] - zg[k0 // GS])
    expect = np.zeros((m, n), dtype=np.float16)
    expect[:, n0] = (x[:, k0].astype(np.float64) * w).astype(np.float16)
    assert np.array_equal(y.view(np.uint16), expect.view(np.uint16))


@pytest.mark.parametrize("lin_idx", range(4))
def test_layer_linears_m16_group_32(lib, lin_idx):
    """The four linears of the 4B-class layer at M = 16 with group-32 weights."""
    k_in, n_out = [(l.k_in, l.n_out) for l in gen.LAYER][lin_idx]
    rng = np.random.default_rng(88 + lin_idx)
    lin = gen.qlinear(rng, k_in, n_out, group_size=GS)
    x = gen.activations(rng, 16, k_in)
    alpha = gen.chain_alpha(k_in)
    y = run_gemm(lib, x, lin, alpha=alpha)
    check_gemm(y, og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros, alpha=alpha, group_size=GS),
               f"g32 layer {k_in}->{n_out}")


def test_deterministic_and_shared_workspace_group_32(lib):
    """Split-K at group size 32 on a workspace shared with group-128 calls: repeated calls are
    bit-identical and the arrival counters are left at zero."""
    import torch
    rng = np.random.default_rng(41)
    k, n = 9728, 2560
    lin32 = gen.qlinear(rng, k, n, group_size=GS)
    lin128 = gen.qlinear(rng, k, n)
    x = gen.activations(rng, 16, k)
    ws = lib.new_workspace(lib.gemm_workspace_size(16, n, k))
    a = run_gemm(lib, x, lin32, ws=ws)
    y128 = host(lib.w4a16_gemm(dev(x), dev(lin128.qweight), dev(lin128.scales), dev(lin128.qzeros),
                               workspace=ws))
    b = run_gemm(lib, x, lin32, ws=ws)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    check_gemm(y128, og.w4a16_gemm(x, lin128.qweight, lin128.scales, lin128.qzeros), "g128 shared")
    assert int(torch.count_nonzero(ws[:65536])) == 0
