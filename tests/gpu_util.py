"""Shared helpers for the GPU parity tests: uploads and the grading rules.

Grading (tolerances of the workload definition):
  G1  W4A16 linear, stage-wise: rel-L2 <= 1e-3 and max-abs <= 1e-2 * rms(ref)
      against the fp64 oracle on the same fp16 input.
  G2  lm_head argmax, stage-wise: ids bit-exact on every row whose oracle
      top-2 margin exceeds 1e-2; on the other rows the GPU's id must be a
      valid answer (its oracle logit within 1e-2 of the row maximum).
  G3  acceptance, free-running: accepted lengths and emitted tokens bit-exact
      whenever every row the decision reads has margin > 1e-2.
  G4  greedy verify alone: bit-exact, always.
"""
import sys

import numpy as np

REL_L2 = 1e-3
MAX_ABS_FRAC = 1e-2
MARGIN = 1e-2


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.detach().cpu().numpy()


def check_gemm(y_gpu, y64, what=""):
    """G1.  Returns (rel_l2, maxabs/rms)."""
    y = np.asarray(y_gpu, dtype=np.float64)
    ref = np.asarray(y64, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    nref = np.linalg.norm(ref)
    rms = nref / np.sqrt(ref.size) if ref.size else 0.0
    if nref == 0:
        assert np.max(np.abs(y)) == 0, f"{what}: expected zeros"
        return 0.0, 0.0
    rel = np.linalg.norm(y - ref) / nref
    mx = np.max(np.abs(y - ref)) / rms
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS_FRAC, f"{what}: max-abs/rms {mx:.3e} > {MAX_ABS_FRAC}"
    return rel, mx


def check_argmax(ids_gpu, logits64, what=""):
    """G2 against full oracle logits [M, V].  Returns the number of low-margin rows."""
    from oracle import lmhead
    t, top, margin = lmhead.argmax_margin(logits64)
    ids = np.asarray(ids_gpu, dtype=np.int64)
    sure = margin > MARGIN
    bad = np.flatnonzero(sure & (ids != t))
    assert bad.size == 0, f"{what}: argmax differs on clear rows {bad[:8]} " \
                          f"(gpu {ids[bad[:8]]}, oracle {t[bad[:8]]}, margin {margin[bad[:8]]})"
    rows = np.flatnonzero(~sure)
    for m in rows:
        v = ids[m]
        assert 0 <= v < logits64.shape[1], f"{what}: id {v} out of range"
        assert logits64[m, v] >= top[m] - MARGIN - 1e-9, f"{what}: row {m} id {v} not near-max"
    return int(rows.size), t, top, margin
