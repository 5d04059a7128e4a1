"""The free-running verify step (oracle; test infrastructure only).

One verify step as the results page (section 3) describes it: the target runs
its linears over the block of K+1 rows, its 8-bit lm_head gives the greedy
token of every row, and greedy acceptance keeps the longest matching draft
prefix plus the bonus token.

Readings where the page is silent about the model between linears: each
linear reads the first k_in columns of the previous fp16 output (the O
projection reads 4096 of the fused QKV's 6144 columns, the down projection
9728 of gate+up's 19456); no attention or activation function is modelled.
Every linear output is rounded to fp16 (the A16 storage point).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import gemm, lmhead, quant, verify


def run_chain(x, linears, plan, workers: int = 1, keep_outputs: bool = True):
    """fp16 output of the chain, plus every linear's fp16 output.

    ``linears``: objects with qweight/scales/qzeros; ``plan``: (k_in, n_out, alpha).
    Dequantised weights do not depend on the activations, so with ``workers``
    > 1 they are produced ``workers`` linears at a time on a thread pool; the
    products then run in chain order, each exactly as ``gemm.w4a16_gemm``.
    """
    h = np.asarray(x, dtype=np.float16)
    outs = []
    pairs = list(zip(linears, plan))
    with ThreadPoolExecutor(max_workers=max(1, workers)) as pool:
        for lo in range(0, len(pairs), max(1, workers)):
            window = pairs[lo:lo + max(1, workers)]
            ws = list(pool.map(lambda p: quant.dequantize(p[0].qweight, p[0].scales, p[0].qzeros),
                               window))
            for w, (_, (k_in, n_out, alpha)) in zip(ws, window):
                y64 = alpha * (h[:, :k_in].astype(np.float64) @ w)
                h = gemm.to_fp16(y64)
                assert h.shape[1] == n_out
                if keep_outputs:
                    outs.append(h)
            del ws
    return h, outs


def verify_step(x, linears, plan, lm_w, lm_s, draft_ids, batch: int, k: int, workers: int = 1):
    """Free-running step: returns dict with h, target ids, margins, accepted lengths, tokens."""
    h, _ = run_chain(x, linears, plan, workers=workers, keep_outputs=False)
    t, top, margin = lmhead.lmhead_argmax(h, lm_w, lm_s)
    tt = t.reshape(batch, k + 1)
    acc, out = verify.greedy_verify(tt, np.asarray(draft_ids).reshape(batch, k), lm_w.shape[0])
    return {"h": h, "target_ids": t, "max_logits": top, "margin": margin,
            "accepted_len": acc, "out_tokens": out,
            "verified_tokens": verify.verified_tokens(acc)}
