"""A verify step of team #5's target (results page, section 5: W4A16 with
group size 32, first and last layers and the lm_head in fp16; n-gram drafts
at K = 23, section 3) on the GPU against the oracle: every linear stage-wise
(G1), the fp16 lm_head's argmax on the GPU's own hidden rows (G2) and the
fused greedy verify on the GPU's target ids (G4), on a reduced target of four
layers with the first and last in fp16."""
import numpy as np
import pytest

import gen
from oracle import gemm as og, lmhead as olm, verify as over
from tests.gpu_util import check_argmax, check_gemm, dev, host, log

pytestmark = pytest.mark.gpu


def device_step(tg):
    from w4a16_speculative_verify_amd.step import DeviceLinear, VerifyStep
    lins = []
    for l in tg.linears:
        if l.w16 is not None:
            lins.append(DeviceLinear(None, None, None, l.k, l.n, l.alpha, w16=dev(l.w16)))
        else:
            lins.append(DeviceLinear(dev(l.q.qweight), dev(l.q.scales), dev(l.q.qzeros), l.k, l.n,
                                     l.alpha, group_size=gen.G32_GROUP))
    return VerifyStep(lins, dev(tg.lm_w16), None, tg.m, 1, tg.k_draft)


def test_g32_target_step_stagewise_and_head():
    import torch
    tg = gen.make_g32_target(layers=4, vocab=4096)
    assert [l.w16 is not None for l in tg.linears] == [True] * 4 + [False] * 8 + [True] * 4
    step = device_step(tg)
    h = dev(tg.x)
    worst = 0.0
    for i, (l, y) in enumerate(zip(tg.linears, step.out)):
        from w4a16_speculative_verify_amd import f16_gemm, w4a16_gemm
        if l.w16 is not None:
            f16_gemm(h[:, :l.k], step.linears[i].w16, alpha=l.alpha, out=y, workspace=step.workspace)
        else:
            w4a16_gemm(h[:, :l.k], step.linears[i].qweight, step.linears[i].scales,
                       step.linears[i].qzeros, alpha=l.alpha, out=y, workspace=step.workspace,
                       group_size=gen.G32_GROUP)
        torch.cuda.synchronize()
        x_in = host(h[:, :l.k])
        ref = og.f16_linear(x_in, l.w16, l.alpha) if l.w16 is not None else \
            og.w4a16_gemm(x_in, l.q.qweight, l.q.scales, l.q.qzeros, l.alpha, group_size=gen.G32_GROUP)
        rel, _ = check_gemm(host(y), ref, f"linear {i}")
        worst = max(worst, rel)
        h = y
    log(f"  g32 target stage-wise worst rel-L2 {worst:.2e}")
    # the fused head on the GPU's own final rows, with planted acceptance
    hh = host(h)
    t_ref, _, _ = olm.lmhead_argmax_f16(hh, tg.lm_w16)
    rng = np.random.default_rng(5)
    drafts = gen.drafts_with_prefix(rng, t_ref, tg.k_draft, 4096, 11)[None, :]
    ids, _, acc, out = step.head(h, dev(drafts))
    torch.cuda.synchronize()
    check_argmax(host(ids), olm.logits_f16(hh, tg.lm_w16), "g32 target head")
    acc_g, out_g = over.greedy_verify(host(ids).reshape(1, -1), drafts, 4096)
    assert np.array_equal(host(acc), acc_g.astype(np.int32)) and np.array_equal(host(out), out_g)


def test_g32_target_step_graph_replays_match_eager():
    import torch
    tg = gen.make_g32_target(seed_offset=1, layers=4, vocab=4096)
    step = device_step(tg)
    x = dev(tg.x)
    drafts = torch.full((1, tg.k_draft), -1, dtype=torch.int32, device="cuda")
    ids, _, _, _ = step(x, drafts)
    eager = host(ids).copy()
    h_eager = host(step.out[-1]).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(x, drafts)
    for rep in range(3):
        step.out[-1].zero_()
        step.target_ids.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(step.out[-1]).view(np.uint16), h_eager.view(np.uint16)), rep
        assert np.array_equal(host(step.target_ids), eager), rep
    assert int(torch.count_nonzero(step.workspace[:65536])) == 0
