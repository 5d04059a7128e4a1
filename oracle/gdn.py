"""Committing a recurrent (Gated DeltaNet) state to the accepted prefix
(oracle; test infrastructure only).

Results page, section 3 and the hazards list: most of the target's layers are
Gated DeltaNet, whose recurrent state a rejected speculative draft corrupted
in the serving engine.  The pages name the layer type (their reference [12])
but not its update; the update below is the gated delta rule of the Gated
DeltaNet paper, written from its definition:

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T

with S [dv, dk], k_t [dk] (unit length in the layer), v_t [dv], alpha_t in
(0, 1] the decay gate and beta_t in [0, 1] the write strength.

Reading of the commit (the step after the verify): the verify block holds
the last committed token at position 0 and the K drafts after it; with a_b
accepted drafts, the state that the next block must start from has consumed
positions 0 .. a_b, i.e. a_b + 1 updates of the state committed before the
block.  Rejected positions are never applied, so no rollback is needed.
"""
import numpy as np


def gdn_update(S, k, v, alpha: float, beta: float) -> np.ndarray:
    """One step of the gated delta rule in fp64: alpha * S (I - beta k k^T) + beta v k^T."""
    S = np.asarray(S, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dk = k.shape[0]
    return alpha * S @ (np.eye(dk) - beta * np.outer(k, k)) + beta * np.outer(v, k)


def commit(state, k, v, alpha, beta, accepted_len) -> np.ndarray:
    """fp64 [B, H, dv, dk]: state[b, h] after positions 0 .. accepted_len[b] of the block.

    state [B, H, dv, dk]; k [B, T, H, dk]; v [B, T, H, dv]; alpha, beta [B, T, H];
    accepted_len [B], clamped to [0, T - 1].
    """
    state = np.asarray(state, dtype=np.float64)
    B, H = state.shape[:2]
    T = np.asarray(k).shape[1]
    out = state.copy()
    for b in range(B):
        a = min(max(int(accepted_len[b]), 0), T - 1)
        for h in range(H):
            S = out[b, h]
            for t in range(a + 1):
                S = gdn_update(S, k[b, t, h], v[b, t, h], float(alpha[b, t, h]), float(beta[b, t, h]))
            out[b, h] = S
    return out
