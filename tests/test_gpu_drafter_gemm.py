"""The 4-bit drafter's step through the same W4A16 linear (results page,
section 5: team #3's W4A16 g128 drafter makes each draft step an INT4 GEMM):
stage-wise parity of all 21 linears at M = 16 (the 12800 -> 2560 fusion, then
five layers of the target's linears) against the oracle, and a captured
drafter step that replays bit-identically to the eager one."""
import numpy as np
import pytest

import gen
from oracle import gemm as og
from tests.gpu_util import check_gemm, dev, host, log

pytestmark = pytest.mark.gpu


def drafter_step(wl):
    from w4a16_speculative_verify_amd.step import DeviceLinear, VerifyStep
    lins = [DeviceLinear(dev(l.qweight), dev(l.scales), dev(l.qzeros), k, n, a)
            for l, (k, n, a) in zip(wl.linears, gen.drafter_plan())]
    return VerifyStep(lins, None, None, 16, 1, 15)


def test_drafter_linears_stagewise():
    import torch
    from w4a16_speculative_verify_amd import w4a16_gemm
    wl = gen.make_drafter_workload()
    step = drafter_step(wl)
    rng = np.random.default_rng(3)
    h = dev(wl.x)
    worst = 0.0
    for i, (lin, (k, n, a), y) in enumerate(zip(wl.linears, gen.drafter_plan(), step.out)):
        w4a16_gemm(h[:, :k], step.linears[i].qweight, step.linears[i].scales,
                   step.linears[i].qzeros, alpha=a, out=y, workspace=step.workspace)
        torch.cuda.synchronize()
        x_in, y_g = host(h[:, :k]), host(y)
        if n > 8192:
            cols = np.sort(rng.choice(n, 1024, replace=False))
            ref = og.w4a16_gemm_columns(x_in, lin.qweight, lin.scales, lin.qzeros, cols, a)
            rel, _ = check_gemm(y_g[:, cols], ref, f"drafter linear {i}")
        else:
            ref = og.w4a16_gemm(x_in, lin.qweight, lin.scales, lin.qzeros, a)
            rel, _ = check_gemm(y_g, ref, f"drafter linear {i}")
        worst = max(worst, rel)
        h = y
    log(f"  drafter stage-wise worst rel-L2 {worst:.2e} over {len(wl.linears)} linears")


def test_drafter_step_graph_replays_match_eager():
    import torch
    wl = gen.make_drafter_workload(seed_offset=1)
    step = drafter_step(wl)
    x = dev(wl.x)
    eager = host(step.linears_only(x).clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step.linears_only(x)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint16), eager.view(np.uint16)), rep
    assert int(torch.count_nonzero(step.workspace[:65536])) == 0
