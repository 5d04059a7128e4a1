"""Pins for the oracle's free-running verify step (``oracle/step.py``).

The chain composes pinned pieces; what these tests pin is the composition
itself, each case chosen so that a plausible slip fails it:
  * a permutation chain with mixed widths (384 -> read 256, 512 -> read 384),
    alpha != 1 and a group-size-32 linear: the expected output is the input's
    columns re-indexed by composing the permutations as integer index arrays
    (no matmul), so a transposed weight, a wrong slice (trailing instead of
    leading columns), a dropped or doubled alpha, or a group size taken as 128
    changes the result;
  * closed forms worked by hand for the fp16 storage point between linears and
    for alpha applied before that rounding (not after);
  * verify_step against lm_head argmax and greedy acceptance composed by hand,
    with drafts whose accepted length is planted.
"""
import numpy as np

import gen
from oracle import gemm, lmhead, step, verify


class _Lin:
    def __init__(self, q, z, s, group_size):
        self.qweight = gen.pack_int4_along_k(q)
        self.qzeros = gen.pack_int4_along_n(z)
        self.scales = np.asarray(s, dtype=np.float16)
        self.group_size = group_size


def _selection_linear(k, n, src, value_code, group_size, rng):
    """W[k, n] with W[src[j], j] = 1 for every column j (src: input index per
    output column); every group g gets its own zero-point and the encoding
    q - z = c_g, s = 1 / c_g with c_g in {1, 2, 4} (exact in fp16).
    ``value_code`` (per column, 1 or 2) multiplies the selected weight: columns
    the next linear must not read carry twice the value (exact in fp16)."""
    groups = k // group_size
    c = np.array([1, 2, 4])[np.arange(groups) % 3]
    z = rng.integers(0, 4, size=(groups, n))
    q = np.repeat(z, group_size, axis=0).copy()
    s = np.empty((groups, n), dtype=np.float64)
    for g in range(groups):
        s[g, :] = 1.0 / c[g]
    for j in range(n):
        kk = src[j]
        g = kk // group_size
        q[kk, j] = z[g, j] + c[g] * value_code[j]
    assert q.max() < 16
    return _Lin(q, z, s, group_size)


def _permutation_chain():
    rng = np.random.default_rng(2024)
    # widths: x 256 -> L0 384 (next reads 256) -> L1 256 -> L2 512 (next reads 384) -> L3 256
    specs = [(256, 384, 256, 1.0, 128), (256, 256, 256, 2.0, 128),
             (256, 512, 384, 0.5, 32), (384, 256, 256, 1.0, 128)]
    lins, plan, srcs, codes = [], [], [], []
    for (k, n, read_next, alpha, gs) in specs:
        src = rng.integers(0, k, size=n)
        src[:read_next] = rng.permutation(k)[:read_next] if read_next <= k else \
            np.concatenate([rng.permutation(k), rng.integers(0, k, read_next - k)])
        code = np.where(np.arange(n) < read_next, 1, 2)
        lin = _selection_linear(k, n, src, code, gs, rng)
        # alpha * s * (q - z) must be 1 on the selected entries: fold 1/alpha into s
        lin.scales = (lin.scales.astype(np.float64) / alpha).astype(np.float16)
        lins.append(lin)
        plan.append((k, n, alpha))
        srcs.append(src)
        codes.append(code)
    return lins, plan, srcs, codes


def test_permutation_chain_with_mixed_widths_is_bit_exact():
    lins, plan, srcs, codes = _permutation_chain()
    x = gen.activations(np.random.default_rng(7), 5, 256)
    h, outs = step.run_chain(x, lins, plan)
    # expected by index composition: output j of a linear is value_code[j] * input[src[j]]
    cur = x.astype(np.float64)
    for (k, n, alpha), src, code, got in zip(plan, srcs, codes, outs):
        cur = cur[:, :k][:, src] * code[None, :]
        assert np.array_equal(got.astype(np.float64), cur)
    assert h.shape == (5, 256)
    assert np.array_equal(h, outs[-1])


def test_trailing_columns_are_never_read():
    """The columns past the next linear's k_in carry doubled values; changing what
    they hold must leave the chain's output unchanged."""
    lins, plan, _, _ = _permutation_chain()
    x = gen.activations(np.random.default_rng(8), 3, 256)
    h_ref, outs = step.run_chain(x, lins, plan)
    # a chain whose first linear writes different values into the unread columns
    rng = np.random.default_rng(99)
    k, n, alpha = plan[0]
    q = gen.pack_int4_along_k(rng.integers(0, 16, size=(k, n)))
    w_keep = lins[0]
    mixed = _Lin(np.zeros((k, n), np.int64), np.zeros((k // 128, n), np.int64),
                 np.ones((k // 128, n)), 128)
    mixed.qweight = w_keep.qweight.copy()
    mixed.qweight[:, plan[1][0]:] = q[:, plan[1][0]:]
    mixed.qzeros, mixed.scales = w_keep.qzeros, w_keep.scales
    h2, outs2 = step.run_chain(x, [mixed] + lins[1:], plan)
    assert not np.array_equal(outs2[0], outs[0])
    assert np.array_equal(h2, h_ref)


def test_fp16_storage_point_between_linears():
    """Hand-worked: linear 0 gives columns (1 + 2^-11, 1); 1 + 2^-11 lies halfway
    between the fp16 neighbours 1 and 1 + 2^-10 and rounds (to even) to 1.
    Linear 1 forms 1024 * col0 - 1024 * col1 (s = 256, q - z = +4 and -4), which
    is 0 exactly; without the fp16 storage point it would be 1024 * 2^-11 = 0.5."""
    k = 128
    x = np.zeros((1, k), dtype=np.float16)
    x[0, 0] = 1.0
    x[0, 1] = 2.0 ** -11
    q0 = np.zeros((k, k), np.int64)
    q0[0, 0] = q0[1, 0] = 1          # col 0 = x0 + x1
    q0[0, 1] = 1                     # col 1 = x0
    l0 = _Lin(q0, np.zeros((1, k), np.int64), np.ones((1, k)), 128)
    n = 8
    z1 = np.full((1, n), 8, np.int64)
    q1 = np.full((k, n), 8, np.int64)
    q1[0, 0], q1[1, 0] = 12, 4
    l1 = _Lin(q1, z1, np.full((1, n), 256.0), 128)
    h, outs = step.run_chain(x, [l0, l1], [(k, k, 1.0), (k, n, 1.0)])
    assert outs[0][0, 0] == np.float16(1.0) and outs[0][0, 1] == np.float16(1.0)
    assert h[0, 0] == 0.0
    unrounded = np.zeros((1, k))
    unrounded[0, 0], unrounded[0, 1] = 1.0 + 2.0 ** -11, 1.0
    assert gemm.w4a16_gemm(unrounded, l1.qweight, l1.scales, l1.qzeros)[0, 0] == 0.5


def test_alpha_is_applied_before_the_rounding():
    """Hand-worked: the accumulator is 1 + 2^-11 and alpha = 3, so
    alpha * acc = 3 + 3 * 2^-11 = 3.00146484375, above the midpoint 3 + 2^-10 of
    the fp16 neighbours 3 and 3 + 2^-9: it rounds to 3 + 2^-9 = 3.001953125.
    Rounding before scaling would give 3 * fp16(1 + 2^-11) = 3."""
    k, n = 128, 8
    x = np.zeros((1, k), dtype=np.float16)
    x[0, 0] = 1.0
    x[0, 1] = 2.0 ** -11
    q = np.zeros((k, n), np.int64)
    q[0, :] = q[1, :] = 1
    lin = _Lin(q, np.zeros((1, n), np.int64), np.ones((1, n)), 128)
    h, _ = step.run_chain(x, [lin], [(k, n, 3.0)])
    assert h[0, 0] == np.float16(3.001953125)
    assert float(h[0, 0]) == 3.0 + 2.0 ** -9


def test_chain_matches_composition_of_pinned_functions():
    rng = np.random.default_rng(31)
    shapes = [(256, 384, 0.7, 128), (256, 256, 1.3, 32), (256, 512, 0.9, 128), (384, 128, 1.1, 32)]
    lins, plan = [], []
    for k, n, a, gs in shapes:
        lins.append(gen.qlinear(rng, k, n, gs))
        plan.append((k, n, a))
    x = gen.activations(rng, 6, 256)
    h, outs = step.run_chain(x, lins, plan)
    cur = x
    for lin, (k, n, a), got in zip(lins, plan, outs):
        cur = gemm.to_fp16(gemm.w4a16_gemm(cur[:, :k], lin.qweight, lin.scales, lin.qzeros, a,
                                           lin.group_size))
        assert np.array_equal(got, cur)
    assert np.array_equal(h, cur)


def test_verify_step_composes_head_argmax_and_acceptance():
    rng = np.random.default_rng(41)
    batch, k_draft, v = 2, 5, 97
    m = batch * (k_draft + 1)
    shapes = [(256, 384, 0.8), (256, 256, 1.2)]
    lins = [gen.qlinear(rng, k, n) for k, n, _ in shapes]
    plan = list(shapes)
    x = gen.activations(rng, m, 256)
    lm_w = gen.lmhead_weights(rng, v, 256)
    lm_s = gen.lmhead_scales(rng, v)
    h, _ = step.run_chain(x, lins, plan)
    t, top, margin = lmhead.lmhead_argmax(h, lm_w, lm_s)
    tt = t.reshape(batch, k_draft + 1)
    planted = [3, 0]
    drafts = np.full((batch, k_draft), -1, dtype=np.int64)
    for b, r in enumerate(planted):
        drafts[b, :r] = tt[b, :r]
        if r < k_draft:
            drafts[b, r] = (tt[b, r] + 1) % v
    res = step.verify_step(x, lins, plan, lm_w, lm_s, drafts, batch, k_draft)
    acc, out = verify.greedy_verify(tt, drafts, v)
    assert np.array_equal(res["h"], h)
    assert np.array_equal(res["target_ids"], t)
    assert np.array_equal(res["margin"], margin)
    assert np.array_equal(res["accepted_len"], acc)
    assert list(res["accepted_len"]) == planted
    assert np.array_equal(res["out_tokens"], out)
    assert res["verified_tokens"] == sum(r + 1 for r in planted)
