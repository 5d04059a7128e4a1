"""GPU parity of the W4A16 linear against the fp64 oracle (G1), plus exact
cases (identity / one-hot weights), strides, determinism and workspace reuse."""
import numpy as np
import pytest

import gen
from oracle import gemm as og
from tests.gpu_util import check_gemm, dev, host, log

pytestmark = pytest.mark.gpu


def run_gemm(w4v, x, lin, alpha=1.0, ws=None, no_ws=False):
    y = w4v.w4a16_gemm(dev(x), dev(lin.qweight), dev(lin.scales), dev(lin.qzeros), alpha=alpha,
                       workspace=ws, no_workspace=no_ws)
    import torch
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("m,k,n", [
    (16, 2560, 2560),          # block linear at M = 16
    (1, 2560, 2560),           # one row: A fragments straight from memory
    (1, 9728, 2560),           # one row, deep K (split across blocks)
    (1, 2560, 19456),          # one row, two tiles per block (LDS-staged activations)
    (5, 384, 200),             # ragged N (not a multiple of 64)
    (16, 1280, 72),
    (21, 1280, 520),           # M = K+1 with K = 20: two m-tiles, ragged rows
    (32, 128, 8),              # single group, narrowest N
    (40, 640, 136),            # more than one m-block
    (16, 9728, 2560),          # deep K (split across blocks)
    (16, 4096, 2560),
    (3, 9728, 1032),
    (33, 256, 200),            # the M >= 33 kernel from one row past a 32-row block
    (130, 384, 136),           # ragged rows and columns
    (300, 1280, 1032),
    (128, 128, 128),           # exactly one tile, one group
])
def test_random_shapes(lib, m, k, n):
    log(f"gemm m={m} k={k} n={n}")
    rng = np.random.default_rng(1000 + m * 7 + k + n)
    lin = gen.qlinear(rng, k, n)
    x = gen.activations(rng, m, k)
    y = run_gemm(lib, x, lin)
    rel, mx = check_gemm(y, og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros), f"{m}x{k}x{n}")
    log(f"  rel-L2 {rel:.2e} max/rms {mx:.2e}")


# ---- M >= 33: the LDS-tiled MFMA kernel (weights dequantised per block tile into LDS as
# fp16(s * (q - z)), split-K with fp32 partials in the workspace for shapes with few tiles)
@pytest.mark.parametrize("m,k,n", [
    (33, 256, 200),            # one ragged row past a 32-row block
    (130, 384, 136),           # ragged rows and columns
    (300, 1280, 1032),
    (128, 128, 128),           # exactly one stage pair, one group
    (168, 2560, 2560),         # the padded verify batch of 8 x 21 rows
    (97, 512, 264),            # 128-row block tiles, ragged rows
    (192, 384, 256),           # 192-row block tiles, every row present
    (600, 1280, 520),
    (257, 4096, 264),          # one row and 8 columns past a 256 x 256 tile
])
def test_mfma_kernel_shapes(lib, m, k, n):
    log(f"gemm mfma m={m} k={k} n={n}")
    rng = np.random.default_rng(7000 + m * 7 + k + n)
    lin = gen.qlinear(rng, k, n)
    x = gen.activations(rng, m, k)
    y = run_gemm(lib, x, lin, alpha=0.75)
    rel, mx = check_gemm(y, og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros, alpha=0.75),
                         f"mfma {m}x{k}x{n}")
    log(f"  rel-L2 {rel:.2e} max/rms {mx:.2e}")


def test_mfma_split_plan_requires_its_workspace(lib):
    """A shape whose plan splits K refuses to run without the workspace the query asks
    for; a shape with one split needs none."""
    import torch
    rng = np.random.default_rng(77)
    k, n, m = 9728, 2560, 168
    assert lib.gemm_workspace_size(m, n, k) > 0
    lin = gen.qlinear(rng, k, n)
    x = gen.activations(rng, m, k)
    with pytest.raises(lib.W4VError):
        run_gemm(lib, x, lin, no_ws=True)
    m2, k2, n2 = 4096, 256, 2048                 # 16 x 8 tiles over 4 stages: no split
    assert lib.gemm_workspace_size(m2, n2, k2) == 0
    lin2 = gen.qlinear(rng, k2, n2)
    x2 = gen.activations(rng, m2, k2)
    y2 = run_gemm(lib, x2, lin2, no_ws=True)
    check_gemm(y2, og.w4a16_gemm(x2, lin2.qweight, lin2.scales, lin2.qzeros), "no split")


@pytest.mark.parametrize("enc", range(3))
@pytest.mark.parametrize("m", [1, 16, 21, 64, 200, 640])
def test_identity_weights_bit_exact(lib, enc, m):
    n = 512
    eye = np.eye(n, dtype=np.int64)
    g = n // 128
    q, z, s = [
        (eye, np.zeros((g, n), np.int64), np.ones((g, n), np.float16)),
        (8 + eye, np.full((g, n), 8, np.int64), np.ones((g, n), np.float16)),
        (7 + 2 * eye, np.full((g, n), 7, np.int64), np.full((g, n), 0.5, np.float16)),
    ][enc]
    lin = gen.QLinear(gen.pack_int4_along_k(q), s, gen.pack_int4_along_n(z), n, n)
    x = gen.activations(np.random.default_rng(enc), m, n)
    y = run_gemm(lib, x, lin)
    assert np.array_equal(y.view(np.uint16), x.view(np.uint16))


def test_one_hot_weight(lib):
    k, n, m = 1024, 264, 16
    k0, n0 = 517, 203
    q = np.full((k, n), 5, dtype=np.int64)
    z = np.full((k // 128, n), 5, dtype=np.int64)
    q[k0, n0] = 13                                   # q - z = 8, scale 0.125 -> w = 1
    s = np.full((k // 128, n), 0.125, dtype=np.float16)
    lin = gen.QLinear(gen.pack_int4_along_k(q), s, gen.pack_int4_along_n(z), k, n)
    x = gen.activations(np.random.default_rng(9), m, k)
    y = run_gemm(lib, x, lin)
    expect = np.zeros((m, n), dtype=np.float16)
    expect[:, n0] = x[:, k0]
    assert np.array_equal(y.view(np.uint16), expect.view(np.uint16))


def test_extreme_codes_and_alpha(lib):
    # q - z at +-15 everywhere with alternating signs, alpha != 1
    k, n, m = 768, 128, 16
    rng = np.random.default_rng(4)
    q = np.where(rng.random((k, n)) < 0.5, 0, 15)
    z = np.where(rng.random((k // 128, n)) < 0.5, 0, 15)
    s = gen.group_scales(rng, k // 128, n)
    lin = gen.QLinear(gen.pack_int4_along_k(q), s, gen.pack_int4_along_n(z), k, n)
    x = gen.activations(rng, m, k)
    y = run_gemm(lib, x, lin, alpha=0.37)
    check_gemm(y, og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros, alpha=0.37), "extreme")


def test_strided_input_and_output(lib):
    import torch
    rng = np.random.default_rng(12)
    k, n, m = 4096, 2560, 16
    lin = gen.qlinear(rng, k, n)
    wide = gen.activations(rng, m, 6144)               # O reads 4096 of QKV's 6144 columns
    out_wide = torch.full((m, 3000), 7.0, dtype=torch.float16, device="cuda")
    out = out_wide[:, 200:200 + n]
    lib.w4a16_gemm(dev(wide)[:, :k], dev(lin.qweight), dev(lin.scales), dev(lin.qzeros), out=out)
    torch.cuda.synchronize()
    full = host(out_wide)
    check_gemm(full[:, 200:200 + n], og.w4a16_gemm(wide[:, :k], lin.qweight, lin.scales, lin.qzeros),
               "strided")
    assert np.all(full[:, :200] == 7.0) and np.all(full[:, 200 + n:] == 7.0)


@pytest.mark.parametrize("k,n", [(9728, 2560), (4096, 2560), (2560, 6144)])
def test_deterministic_and_workspace_reuse(lib, k, n):
    rng = np.random.default_rng(k + n)
    lin = gen.qlinear(rng, k, n)
    x1 = gen.activations(rng, 16, k)
    x2 = gen.activations(rng, 16, k)
    need = lib.gemm_workspace_size(16, n, k)
    ws = lib.new_workspace(need) if need else None
    a = run_gemm(lib, x1, lin, ws=ws)
    b = run_gemm(lib, x2, lin, ws=ws)           # counters re-armed by the kernel
    c = run_gemm(lib, x1, lin, ws=ws)
    assert np.array_equal(a.view(np.uint16), c.view(np.uint16))
    check_gemm(b, og.w4a16_gemm(x2, lin.qweight, lin.scales, lin.qzeros), "reuse")
    if ws is not None:
        import torch
        assert int(torch.count_nonzero(ws[:65536])) == 0     # counters back at zero


def test_workspace_shared_across_shapes(lib):
    """One workspace for linears of different shapes, in chain order (as a verify step does)."""
    rng = np.random.default_rng(21)
    shapes = [(2560, 6144), (4096, 2560), (2560, 19456), (9728, 2560), (2560, 6144)]
    lins = [gen.qlinear(rng, k, n) for k, n in shapes]
    need = max(lib.gemm_workspace_size(16, n, k) for k, n in shapes)
    ws = lib.new_workspace(need)
    for rep in range(2):
        for lin, (k, n) in zip(lins, shapes):
            x = gen.activations(rng, 16, k)
            y = run_gemm(lib, x, lin, ws=ws)
            check_gemm(y, og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros), f"{k}->{n}")


@pytest.mark.parametrize("lin_idx", range(4))
def test_layer_linears_m16(lib, lin_idx):
    """The four linears of the 4B-class layer at the verify block size M = 16."""
    wl = gen.make_workload(3, layers=1, vocab=0)
    k_in, n_out, alpha = gen.chain_plan(wl.cfg)[lin_idx]
    lin = wl.linears[lin_idx]
    x = gen.activations(np.random.default_rng(77 + lin_idx), 16, k_in)
    log(f"layer linear {lin_idx}: {k_in}->{n_out}")
    y = run_gemm(lib, x, lin, alpha=alpha)
    check_gemm(y, og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros, alpha=alpha), "layer")


@pytest.mark.parametrize("shape", [(2560, 6144), (4096, 2560), (2560, 19456), (9728, 2560)])
def test_padded_verify_block_full(lib, shape):
    """The batched verify block (8 sequences x 21 rows): every output of every layer linear."""
    k, n = shape
    rng = np.random.default_rng(168 + k + n)
    lin = gen.qlinear(rng, k, n)
    x = gen.activations(rng, 168, k)
    a = gen.chain_alpha(k)
    y = run_gemm(lib, x, lin, alpha=a)
    rel, mx = check_gemm(y, og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros, alpha=a),
                         f"m=168 {k}->{n}")
    log(f"  m=168 {k}->{n}: rel-L2 {rel:.2e} max/rms {mx:.2e}")


@pytest.mark.parametrize("m", [2048, 8192])
@pytest.mark.parametrize("shape", [(2560, 19456), (9728, 2560)])
def test_prefill_full_output(lib, m, shape):
    """Prefill shapes (M = 2048, 8192): every output element against the fp64 oracle of
    the whole product (0.1-0.8 TFLOP of fp64, seconds on the host)."""
    k, n = shape
    wl = gen.make_workload(5, m=m)
    lin = wl.linears[0] if k == 2560 else wl.linears[1]
    x = wl.extra_x[0] if k == 2560 else wl.extra_x[1]
    log(f"prefill m={m} {k}->{n}")
    y = run_gemm(lib, x, lin)
    ref = og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros)
    rel, mx = check_gemm(y, ref, f"m={m} {k}->{n}")
    log(f"  rel-L2 {rel:.2e} max/rms {mx:.2e} over all {m} x {n} outputs")


# ---- M >= 33 path, more shapes (the split and unsplit plans)
@pytest.mark.parametrize("m,k,n", [
    (511, 384, 136),
    (512, 384, 136),           # ragged N
    (600, 1280, 1032),
    (1000, 128, 8),            # one group, narrowest N
    # 3 x 89 = 267 tiles on 256 CUs: 256 whole tiles, the last 11 split 8 ways, ragged
    # rows (88 of the last row block) and columns (8 of the last column block)
    (600, 2048, 22536),
])
def test_mfma_path_shapes(lib, m, k, n):
    log(f"gemm m={m} k={k} n={n}")
    rng = np.random.default_rng(3000 + m + k + n)
    lin = gen.qlinear(rng, k, n)
    x = gen.activations(rng, m, k)
    y = run_gemm(lib, x, lin, alpha=0.75)
    rel, mx = check_gemm(y, og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros, alpha=0.75),
                         f"{m}x{k}x{n}")
    log(f"  rel-L2 {rel:.2e} max/rms {mx:.2e}")


def test_mfma_path_strided_and_shared_workspace(lib):
    """Row-strided x and y at M = 700, then M = 16 split-K calls on the same workspace: the
    counter prefix the skinny split-K path relies on is left at zero by the M >= 33 path."""
    import torch
    rng = np.random.default_rng(31)
    k, n, m = 1024, 520, 700
    lin = gen.qlinear(rng, k, n)
    wide = gen.activations(rng, m, 1536)
    need = max(lib.gemm_workspace_size(m, n, k), lib.gemm_workspace_size(16, 2560, 9728))
    ws = lib.new_workspace(need)
    out_wide = torch.full((m, 800), 7.0, dtype=torch.float16, device="cuda")
    out = out_wide[:, 96:96 + n]               # 192 bytes in: 16-byte aligned
    lib.w4a16_gemm(dev(wide)[:, :k], dev(lin.qweight), dev(lin.scales), dev(lin.qzeros), out=out,
                   workspace=ws)
    torch.cuda.synchronize()
    full = host(out_wide)
    check_gemm(full[:, 96:96 + n], og.w4a16_gemm(wide[:, :k], lin.qweight, lin.scales, lin.qzeros),
               "strided m=700")
    assert np.all(full[:, :96] == 7.0) and np.all(full[:, 96 + n:] == 7.0)
    assert int(torch.count_nonzero(ws[:65536])) == 0
    lin2 = gen.qlinear(rng, 9728, 2560)
    for _ in range(2):
        x2 = gen.activations(rng, 16, 9728)
        y2 = run_gemm(lib, x2, lin2, ws=ws)
        check_gemm(y2, og.w4a16_gemm(x2, lin2.qweight, lin2.scales, lin2.qzeros), "split-K after")
