"""GPU parity of committing a Gated DeltaNet state to the accepted prefix
against the fp64 oracle (fp32 arithmetic: at most 32 steps of a 128-term dot
product and a rank-one update, relative error below 32 * sqrt(128) * 2^-23,
about 4.3e-5), including clamped accepted lengths, both head widths and the
largest block, and the closed loop greedy verify -> commit on the device."""
import numpy as np
import pytest

import gen
from oracle import gdn, verify as over
from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu
TOL = 5e-5


def check_state(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), what
    for idx in np.ndindex(ref.shape[:2]):
        g, r = got[idx], ref[idx]
        rel = np.linalg.norm(g - r) / np.linalg.norm(r)
        mx = np.max(np.abs(g - r)) / (np.linalg.norm(r) / np.sqrt(r.size))
        assert rel <= TOL and mx <= 10 * TOL, f"{what} {idx}: rel-L2 {rel:.2e}, max/rms {mx:.2e}"


@pytest.mark.parametrize("b,t,h,d,acc", [
    (3, 16, 4, 128, [0, 15, 7]),
    (2, 16, 3, 64, [3, 11]),
    (1, 1, 2, 128, [0]),                 # T = 1: the last committed token only
    (2, 32, 2, 128, [31, 20]),           # the largest block
    (3, 21, 2, 128, [-4, 99, 5]),        # clamped to [0, T - 1]
])
def test_commit_matches_oracle(lib, b, t, h, d, acc):
    import torch
    rng = np.random.default_rng(b * 100 + t * 10 + h + d)
    S, k, v, al, be = gen.gdn_inputs(rng, b, t, h, d, d)
    acc = np.asarray(acc, np.int32)
    s_d = dev(S)
    lib.gdn_state_commit(s_d, dev(k), dev(v), dev(al), dev(be), dev(acc))
    torch.cuda.synchronize()
    check_state(host(s_d), gdn.commit(S, k, v, al, be, acc), f"commit b={b} t={t} h={h} d={d}")


def test_verify_then_commit_on_device(lib):
    """greedy_verify's accepted lengths feed the commit without a host round trip, over three
    blocks in a row, against the same rounds through the oracle."""
    import torch
    rng = np.random.default_rng(7)
    B, K, H, V = 4, 15, 8, 1000
    S, _, _, _, _ = gen.gdn_inputs(rng, B, 1, H)
    s_d = dev(S)
    ref = S.astype(np.float64)
    for r in range(3):
        _, k, v, al, be = gen.gdn_inputs(rng, B, K + 1, H)
        tgt = rng.integers(0, V, (B, K + 1)).astype(np.int32)
        drafts = np.stack([gen.drafts_with_prefix(rng, tgt[i], K, V, int(rng.integers(0, K + 1)))
                           for i in range(B)])
        acc_d, _ = lib.greedy_verify(dev(tgt), dev(drafts), V)
        lib.gdn_state_commit(s_d, dev(k), dev(v), dev(al), dev(be), acc_d)
        torch.cuda.synchronize()
        acc_o, _ = over.greedy_verify(tgt, drafts, V)
        assert np.array_equal(host(acc_d), acc_o.astype(np.int32)), r
        ref = gdn.commit(ref, k, v, al, be, acc_o)
        check_state(host(s_d), ref, f"round {r}")
    log(f"  verify -> commit: 3 rounds x {B} sequences x {H} heads")
