"""The free-running verify step (oracle; test infrastructure only).

One verify step as the results page ("Efficient LLM Challenge Results",
section 3) describes it: the target runs its linears over the block of K+1
rows, its 8-bit lm_head gives the greedy token of every row, and greedy
acceptance keeps the longest matching draft prefix plus the bonus token.

Readings where the page is silent about the model between linears: each
linear reads the first k_in columns of the previous fp16 output (the O
projection reads 4096 of the fused QKV's 6144 columns, the down projection
9728 of gate+up's 19456); no attention or activation function is modelled.
Every linear output is rounded to fp16 (the A16 storage point), after its
epilogue scale alpha.

The chain is nothing but the pinned pieces composed in order:
``gemm.w4a16_gemm`` (with each linear's own group size), then
``gemm.to_fp16``; the step adds ``lmhead.lmhead_argmax`` and
``verify.greedy_verify``.  ``tests/test_oracle_step.py`` pins the
composition (slicing, alpha before the rounding, the rounding itself, the
group size) with closed forms and permutation chains.
"""
import numpy as np

from . import gemm, lmhead, quant, verify


def run_chain(x, linears, plan, keep_outputs: bool = True):
    """fp16 output of the chain, plus every linear's fp16 output.

    ``linears``: objects with qweight / scales / qzeros (and optionally
    ``group_size``, 128 when absent); ``plan``: one (k_in, n_out, alpha) per
    linear.  Linear i computes fp16(alpha_i * h[:, :k_in_i] @ W_i) from the
    previous fp16 output h (x for the first).
    """
    h = np.asarray(x, dtype=np.float16)
    outs = []
    for lin, (k_in, n_out, alpha) in zip(linears, plan):
        g = getattr(lin, "group_size", quant.GROUP_SIZE)
        y64 = gemm.w4a16_gemm(h[:, :k_in], lin.qweight, lin.scales, lin.qzeros, alpha, g)
        h = gemm.to_fp16(y64)
        if h.shape[1] != n_out:
            raise ValueError(f"linear produced {h.shape[1]} columns, plan says {n_out}")
        if keep_outputs:
            outs.append(h)
    return h, outs


def verify_step(x, linears, plan, lm_w, lm_s, draft_ids, batch: int, k: int):
    """Free-running step: returns dict with h, target ids, margins, accepted lengths, tokens."""
    h, _ = run_chain(x, linears, plan, keep_outputs=False)
    t, top, margin = lmhead.lmhead_argmax(h, lm_w, lm_s)
    tt = t.reshape(batch, k + 1)
    acc, out = verify.greedy_verify(tt, np.asarray(draft_ids).reshape(batch, k), lm_w.shape[0])
    return {"h": h, "target_ids": t, "max_logits": top, "margin": margin,
            "accepted_len": acc, "out_tokens": out,
            "verified_tokens": verify.verified_tokens(acc)}
