"""int4 unpacking and group-wise dequantisation (oracle; test infrastructure only).

The results page (section 3 and section 5) fixes the format as W4A16 with
group size 128 along the reduction dimension.  Readings where it is silent:
  * asymmetric dequantisation  w = s[g, n] * (q[k, n] - z[g, n]),
    g = floor(k / 128), groups contiguous along k (no act-order permutation);
  * nibble j of a 32-bit word sits at bits 4j..4j+3 (lowest nibble first);
    weights pack 8 consecutive k per word, zero-points 8 consecutive n.
"""
import numpy as np

GROUP_SIZE = 128


def _nibbles(words: np.ndarray) -> list:
    """The eight nibbles (0..15) of each word, read as an unsigned 32-bit value."""
    w = np.asarray(words).view(np.uint32)
    return [((w >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.int16) for j in range(8)]


def unpack_weights(qweight: np.ndarray) -> np.ndarray:
    """int32 [K/8, N] -> int16 [K, N] with q[8i + j, n] = nibble j of word (i, n)."""
    rows, n = qweight.shape
    nib = _nibbles(qweight)
    q = np.empty((rows * 8, n), dtype=np.int16)
    for j in range(8):
        q[j::8, :] = nib[j]
    return q


def unpack_zeros(qzeros: np.ndarray) -> np.ndarray:
    """int32 [G, N/8] -> int16 [G, N] with z[g, 8i + j] = nibble j of word (g, i)."""
    g, cols = qzeros.shape
    nib = _nibbles(qzeros)
    z = np.empty((g, cols * 8), dtype=np.int16)
    for j in range(8):
        z[:, j::8] = nib[j]
    return z


def dequantize(qweight, scales, qzeros, group_size: int = GROUP_SIZE) -> np.ndarray:
    """fp64 [K, N]: W[k, n] = s[g, n] * (q[k, n] - z[g, n]) with g = k // group_size.

    Exact in fp64: the fp16 scale times an integer in [-15, 15] needs at most
    15 significant bits.
    """
    q = unpack_weights(qweight)
    z = unpack_zeros(qzeros)
    k, n = q.shape
    groups = k // group_size
    s = np.asarray(scales).astype(np.float64)
    # view k as (g, k mod group_size) so the per-group s and z broadcast along it
    w = (q.reshape(groups, group_size, n) - z[:, None, :]).astype(np.float64)
    w *= s[:, None, :]
    return w.reshape(k, n)


def dequantize_columns(qweight, scales, qzeros, cols, group_size: int = GROUP_SIZE) -> np.ndarray:
    """Dequantise only the listed output columns: fp64 [K, len(cols)].

    Same definition as :func:`dequantize`, restricted to a column subset so
    that large matrices can be checked on sampled outputs.
    """
    cols = np.asarray(cols)
    q = unpack_weights(np.asarray(qweight)[:, cols])
    zall = unpack_zeros(qzeros)
    z = zall[:, cols]
    k = q.shape[0]
    g = np.arange(k) // group_size
    s = np.asarray(scales)[:, cols].astype(np.float64)
    return s[g, :] * (q - z[g, :]).astype(np.float64)
