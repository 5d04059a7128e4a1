"""The W4A16 linear (oracle; test infrastructure only).

Results page, section 3: the verify pass runs the target's linears over the
K+1 positions at once (a block of M = K+1 activation rows); the target's
weights are 4-bit with group size 128 and activations stay 16-bit (W4A16).

Definition:  Y[m, n] = alpha * sum_k X[m, k] * W[k, n]  in fp64, where W is
the dequantised weight.  Activations are stored as fp16 between linears, so
the value handed to the next linear is fp16(Y) rounded to nearest even.
``alpha`` is the epilogue scale of the chained workloads (1 for a stand-alone
linear).
"""
import numpy as np

from . import quant


def w4a16_gemm(x, qweight, scales, qzeros, alpha: float = 1.0,
               group_size: int = quant.GROUP_SIZE) -> np.ndarray:
    """fp64 [M, N] = alpha * X64 @ W64."""
    w = quant.dequantize(qweight, scales, qzeros, group_size)
    return alpha * (np.asarray(x).astype(np.float64) @ w)


def w4a16_gemm_columns(x, qweight, scales, qzeros, cols, alpha: float = 1.0,
                       group_size: int = quant.GROUP_SIZE) -> np.ndarray:
    """The same product restricted to output columns ``cols``: fp64 [M, len(cols)]."""
    w = quant.dequantize_columns(qweight, scales, qzeros, cols, group_size)
    return alpha * (np.asarray(x).astype(np.float64) @ w)


def to_fp16(y64: np.ndarray) -> np.ndarray:
    """fp16 storage point: round-to-nearest-even from fp64."""
    return np.asarray(y64, dtype=np.float64).astype(np.float16)


def f16_linear(x, w, alpha: float = 1.0) -> np.ndarray:
    """fp64 [M, N] = alpha * X64 @ W64^T for fp16 weights W [N, K] (one row per output).

    Results page, section 5: team #5 keeps the first two and last two layers
    of its group-size-32 target in half precision; those linears are plain
    fp16 products, W in the [out, in] layout of a dense layer.
    """
    return alpha * (np.asarray(x).astype(np.float64) @ np.asarray(w).astype(np.float64).T)

