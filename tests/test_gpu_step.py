"""End-to-end verify steps on the GPU against the oracle: stage-wise per
linear (G1), lm_head on the GPU's own hidden rows (G2), and the free-running
acceptance (G3) with drafts built from the oracle's own target ids."""
import numpy as np
import pytest

import gen
from oracle import gemm as og, lmhead as olm, step as ostep, verify as over
from tests.gpu_util import MARGIN, check_argmax, check_gemm, dev, host, log

pytestmark = pytest.mark.gpu


def device_step(wl, m=None):
    from w4a16_speculative_verify_amd.step import DeviceLinear, VerifyStep
    cfg = wl.cfg
    plan = gen.chain_plan(cfg)
    lins = [DeviceLinear(dev(l.qweight), dev(l.scales), dev(l.qzeros), k, n, a)
            for l, (k, n, a) in zip(wl.linears, plan)]
    lm_w = dev(wl.lm_w) if wl.lm_w is not None else None
    lm_s = dev(wl.lm_s) if wl.lm_s is not None else None
    return VerifyStep(lins, lm_w, lm_s, m or cfg.m, cfg.batch, cfg.k_draft)


def stagewise(step, wl, sample_cols=None, seed=0):
    """Run the chain linear by linear; check each output against the oracle on
    the GPU's own fp16 input.  Returns the final hidden rows (host)."""
    import torch
    plan = gen.chain_plan(wl.cfg)
    rng = np.random.default_rng(seed)
    h = dev(wl.x)
    worst = 0.0
    for i, (lin, (k, n, a), y) in enumerate(zip(wl.linears, plan, step.out)):
        from w4a16_speculative_verify_amd import w4a16_gemm
        w4a16_gemm(h[:, :k], step.linears[i].qweight, step.linears[i].scales,
                   step.linears[i].qzeros, alpha=a, out=y, workspace=step.workspace)
        torch.cuda.synchronize()
        x_in = host(h[:, :k])
        y_g = host(y)
        if sample_cols:
            cols = np.sort(rng.choice(n, sample_cols, replace=False))
            ref = og.w4a16_gemm_columns(x_in, lin.qweight, lin.scales, lin.qzeros, cols, a)
            rel, _ = check_gemm(y_g[:, cols], ref, f"linear {i}")
        else:
            ref = og.w4a16_gemm(x_in, lin.qweight, lin.scales, lin.qzeros, a)
            rel, _ = check_gemm(y_g, ref, f"linear {i}")
        worst = max(worst, rel)
        h = y
    log(f"  stage-wise worst rel-L2 {worst:.2e} over {len(plan)} linears")
    return host(h)


def free_running(wl, step, min_pinned=1):
    """G3: drafts from the oracle's own free-running target ids (fresh draft stream).
    At least ``min_pinned`` sequences must have every consulted row above the
    margin, so that the comparison decides something."""
    import torch
    cfg = wl.cfg
    plan = gen.chain_plan(cfg)
    ref = ostep.verify_step(wl.x, wl.linears, plan, wl.lm_w, wl.lm_s,
                            np.zeros((cfg.batch, cfg.k_draft), np.int32), cfg.batch, cfg.k_draft)
    t_o, margin = ref["target_ids"], ref["margin"]
    drafts, r = gen.make_drafts(gen.draft_rng(cfg.cid), cfg, t_o)
    a_o, out_o = over.greedy_verify(t_o.reshape(cfg.batch, -1), drafts, cfg.vocab)
    assert np.array_equal(a_o, r)
    t_g, _, acc, out = step(dev(wl.x), dev(drafts))
    torch.cuda.synchronize()
    t_g, acc, out = host(t_g), host(acc), host(out)
    h_g = host(step.out[-1])
    rel_h = np.linalg.norm(h_g.astype(np.float64) - ref["h"].astype(np.float64)) / \
        np.linalg.norm(ref["h"].astype(np.float64))
    pinned = 0
    for b in range(cfg.batch):
        rows = b * (cfg.k_draft + 1) + np.arange(a_o[b] + 1)
        if np.all(margin[rows] > MARGIN):
            assert acc[b] == a_o[b], f"seq {b}: accepted {acc[b]} vs oracle {a_o[b]}"
            assert np.array_equal(out[b], out_o[b])
            pinned += 1
        else:
            first = rows[np.argmax(margin[rows] <= MARGIN)]
            upto = first - b * (cfg.k_draft + 1)
            assert np.array_equal(out[b][:upto], out_o[b][:upto])
    log(f"  free-running: final-h rel-L2 {rel_h:.2e}; {pinned}/{cfg.batch} sequences pinned; "
        f"accepted {acc.tolist()} (oracle {a_o.tolist()})")
    assert pinned >= min_pinned, f"only {pinned} of {cfg.batch} sequences pinned"
    return pinned


def test_c1_block_linear_step(lib):
    wl = gen.make_workload(1)
    step = device_step(wl)
    h = stagewise(step, wl)
    lg = olm.logits(h, wl.lm_w, wl.lm_s)
    import torch
    t_g, _ = lib.w8a16_lmhead_argmax(dev(h), step.lm_w, step.lm_s)
    torch.cuda.synchronize()
    check_argmax(host(t_g), lg, "c1 lm_head")
    free_running(wl, step)


def test_c2_decode_layer(lib):
    wl = gen.make_workload(2)
    step = device_step(wl)
    stagewise(step, wl)
    import torch
    h_g = host(step.linears_only(dev(wl.x)))
    torch.cuda.synchronize()
    h_o, _ = ostep.run_chain(wl.x, wl.linears, gen.chain_plan(wl.cfg))
    rel = np.linalg.norm(h_g.astype(np.float64) - h_o) / np.linalg.norm(h_o.astype(np.float64))
    assert rel < 1e-2, rel
    log(f"  c2 free-running rel-L2 {rel:.2e}")


def test_c3_verify_step(lib):
    """36 layers at M = 16 and the 151,936-word lm_head."""
    log("c3: generating inputs")
    wl = gen.make_workload(3)
    step = device_step(wl)
    log("c3: stage-wise (every output column of all 144 linears)")
    h = stagewise(step, wl)
    lg = olm.logits(h, wl.lm_w, wl.lm_s)
    import torch
    t_g, _ = lib.w8a16_lmhead_argmax(dev(h), step.lm_w, step.lm_s)
    torch.cuda.synchronize()
    low, *_ = check_argmax(host(t_g), lg, "c3 lm_head")
    log(f"  lm_head low-margin rows {low}/16")
    log("c3: free-running oracle chain")
    free_running(wl, step)


def test_c4_padded_batch(lib):
    """8 sequences x 21 rows through one layer, 151,936-word lm_head, K = 20 with -1 padding."""
    wl = gen.make_workload(4)
    step = device_step(wl)
    h = stagewise(step, wl)
    lg = olm.logits(h, wl.lm_w, wl.lm_s)
    import torch
    t_g, _ = lib.w8a16_lmhead_argmax(dev(h), step.lm_w, step.lm_s)
    torch.cuda.synchronize()
    check_argmax(host(t_g), lg, "c4 lm_head")
    free_running(wl, step)
