"""GPU parity of the one-launch chain of W4A16 linears (w4a16_chain): every
intermediate fp16 output is read back from the workspace and checked against
the oracle on the GPU's own input (G1); also determinism, repeated launches,
graph replay and the unprepared-workspace guard."""
import numpy as np
import pytest

import gen
from oracle import gemm as og
from tests.gpu_util import check_gemm, dev, host, log

pytestmark = pytest.mark.gpu

# ChainLinear (w4v_launch.h): 4 pointers, 3 ints, float, 4 ints
_LIN = np.dtype([("out", "<u8"), ("flags", "<u8"), ("sflags", "<u8"), ("partials", "<u8"),
                 ("K", "<i4"), ("N", "<i4"), ("ldo", "<i4"), ("alpha", "<f4"),
                 ("S", "<i4"), ("tiles", "<i4"), ("pad0", "<i4"), ("pad1", "<i4")])


def intermediates(chain):
    """fp16 outputs of linears 0..n-2 as the last launch wrote them."""
    import torch
    torch.cuda.synchronize()
    ws = chain.workspace
    hdr = ws[:256].cpu().numpy()
    n = int(hdr[4:8].view(np.uint32)[0])
    lin_off = int(hdr[48:56].view(np.uint64)[0])
    tab = ws[lin_off:lin_off + n * _LIN.itemsize].cpu().numpy().view(_LIN)
    base = ws.data_ptr()
    outs = []
    for l in range(n - 1):
        ldo, N = int(tab["ldo"][l]), int(tab["N"][l])
        off = int(tab["out"][l]) - base
        buf = ws[off:off + 16 * ldo * 2].view(torch.float16).view(16, ldo)
        outs.append(host(buf[:chain.m, :N]))
    return outs


def build(lins, m, alphas):
    import w4a16_speculative_verify_amd as w4v
    return w4v.Chain([(dev(l.qweight), dev(l.scales), dev(l.qzeros), a)
                      for l, a in zip(lins, alphas)], m)


def check_chain(chain, x, lins, alphas, y, sample_cols=None, seed=0):
    mids = intermediates(chain)
    rng = np.random.default_rng(seed)
    h = x
    worst = 0.0
    for i, (lin, a) in enumerate(zip(lins, alphas)):
        got = mids[i] if i < len(lins) - 1 else y
        xin = h[:, :lin.k]
        if sample_cols and lin.n > sample_cols:
            cols = np.sort(rng.choice(lin.n, sample_cols, replace=False))
            ref = og.w4a16_gemm_columns(xin, lin.qweight, lin.scales, lin.qzeros, cols, a)
            rel, _ = check_gemm(got[:, cols], ref, f"chain linear {i}")
        else:
            rel, _ = check_gemm(got, og.w4a16_gemm(xin, lin.qweight, lin.scales, lin.qzeros, a),
                                f"chain linear {i}")
        worst = max(worst, rel)
        h = got
    return worst


@pytest.mark.parametrize("m", [16, 1, 5])
def test_chain_small(lib, m):
    rng = np.random.default_rng(100 + m)
    shapes = [(256, 208), (128, 1024), (1024, 640), (640, 144), (128, 2560)]
    lins = [gen.qlinear(rng, k, n) for k, n in shapes]
    alphas = [gen.chain_alpha(k) for k, _ in shapes]
    x = gen.activations(rng, m, shapes[0][0])
    chain = build(lins, m, alphas)
    y = host(chain(dev(x)))
    assert chain.error() == 0
    worst = check_chain(chain, x, lins, alphas, y)
    log(f"  chain m={m}: worst stage-wise rel-L2 {worst:.2e}")


def test_chain_single_linear(lib):
    rng = np.random.default_rng(7)
    lin = gen.qlinear(rng, 2560, 2560)
    x = gen.activations(rng, 16, 2560)
    chain = build([lin], 16, [1.0])
    y = host(chain(dev(x)))
    check_gemm(y, og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros), "single")


def test_chain_verify_step_layers(lib):
    """The 36-layer verify-step chain at M = 16: all 144 linears stage-wise (every output
    column), bit-identical repeats, error word clear after several launches."""
    import torch
    log("chain c3: generating")
    wl = gen.make_workload(3, vocab=0)
    plan = gen.chain_plan(wl.cfg)
    lins = wl.linears
    alphas = [a for _, _, a in plan]
    chain = build(lins, 16, alphas)
    xd = dev(wl.x)
    y1 = host(chain(xd))
    y2 = host(chain(xd))
    y3 = host(chain(xd))
    torch.cuda.synchronize()
    assert chain.error() == 0
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    assert np.array_equal(y1.view(np.uint16), y3.view(np.uint16))
    worst = check_chain(chain, wl.x, lins, alphas, y3)
    log(f"  chain c3: worst stage-wise rel-L2 {worst:.2e} over {len(lins)} linears")


def test_chain_matches_per_linear_path_exactly_when_single_split(lib):
    """With K = 1024 every unit has one split: the chain and w4a16_gemm then add the
    same products in a different order only inside the MFMA, so compare to tolerance."""
    rng = np.random.default_rng(11)
    lins = [gen.qlinear(rng, 1024, 1024) for _ in range(3)]
    alphas = [gen.chain_alpha(1024)] * 3
    x = gen.activations(rng, 16, 1024)
    chain = build(lins, 16, alphas)
    y = host(chain(dev(x)))
    check_chain(chain, x, lins, alphas, y)


def test_chain_graph_replay(lib):
    import torch
    rng = np.random.default_rng(13)
    shapes = [(2560, 6144), (4096, 2560), (2560, 19456), (9728, 2560)]
    lins = [gen.qlinear(rng, k, n) for k, n in shapes]
    alphas = [gen.chain_alpha(k) for k, _ in shapes]
    chain = build(lins, 16, alphas)
    xs = [gen.activations(rng, 16, 2560) for _ in range(3)]
    eager = [host(chain(dev(x))) for x in xs]
    xbuf = dev(xs[0])
    ybuf = torch.empty((16, 2560), dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain(xbuf, out=ybuf)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain(xbuf, out=ybuf)
    for rep in range(2):
        for i, x in enumerate(xs):
            xbuf.copy_(dev(x))
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host(ybuf).view(np.uint16), eager[i].view(np.uint16)), (rep, i)
    assert chain.error() == 0


def test_chain_unprepared_workspace_is_refused(lib):
    import ctypes
    import torch
    import w4a16_speculative_verify_amd as w4v
    rng = np.random.default_rng(17)
    lin = gen.qlinear(rng, 256, 256)
    chain = build([lin], 16, [1.0])
    ws = w4v.new_workspace(chain.workspace.numel())          # zeroed, never prepared
    x = dev(gen.activations(rng, 16, 256))
    y = torch.full((16, 256), 3.0, dtype=torch.float16, device="cuda")
    st = w4v.load().w4a16_chain(x.data_ptr(), 256, y.data_ptr(), 256, 16, 256, 256,
                                ctypes.c_void_p(ws.data_ptr()),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    err = int(ws[28:32].cpu().view(torch.int32).item())
    assert err == 2
    assert bool(torch.all(y == 3.0))
    # a prepared workspace with a different shape is refused the same way
    st = w4v.load().w4a16_chain(x.data_ptr(), 256, y.data_ptr(), 256, 8, 256, 256,
                                ctypes.c_void_p(chain.workspace.data_ptr()),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    assert chain.error() == 2
