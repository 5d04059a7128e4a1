"""The entry point that allocates nothing (w4a16_gemm_noalloc) against the
workspace entry point it mirrors: bit-identical outputs on two calls in a
row, the second smaller than the first (the static scratch keeps the first
call's contents), plus G1 parity against the fp64 oracle."""
import numpy as np
import pytest

import gen
from oracle import gemm as og
from tests.gpu_util import check_gemm, dev, host, log

pytestmark = pytest.mark.gpu


def _pair(w4v, x, lin, alpha):
    import torch
    xd, qw, sc, qz = dev(x), dev(lin.qweight), dev(lin.scales), dev(lin.qzeros)
    y_ws = w4v.w4a16_gemm(xd, qw, sc, qz, alpha=alpha)
    y_na = torch.full_like(y_ws, float("nan"))
    w4v.w4a16_gemm_noalloc(xd, qw, sc, qz, alpha=alpha, out=y_na)
    torch.cuda.synchronize()
    return host(y_ws), host(y_na)


@pytest.mark.parametrize("shapes", [
    # split-K skinny plans (tickets + partials), then a smaller one
    ((16, 4096, 2560), (5, 1280, 520)),
    # deep K with many splits, then a one-group shape
    ((16, 9728, 2560), (3, 128, 8)),
    # the M >= 33 kernel with K-split partials in the scratch, then a smaller split plan
    ((168, 2560, 6144), (40, 1280, 136)),
    # whole tiles plus a split tail (256 + 11 x 8), then a fully split plan
    ((600, 2048, 22536), (40, 1280, 136)),
])
def test_noalloc_matches_workspace_entry_point(lib, shapes):
    for i, (m, k, n) in enumerate(shapes):
        log(f"noalloc call {i}: m={m} k={k} n={n}")
        rng = np.random.default_rng(7000 + 13 * i + m + k + n)
        lin = gen.qlinear(rng, k, n)
        x = gen.activations(rng, m, k)
        alpha = 0.75 if i else 1.0
        y_ws, y_na = _pair(lib, x, lin, alpha)
        assert np.array_equal(y_ws.view(np.uint16), y_na.view(np.uint16)), \
            f"call {i}: outputs differ from w4a16_gemm"
        y64 = og.w4a16_gemm(x, lin.qweight, lin.scales, lin.qzeros, alpha)
        check_gemm(y_na, y64, f"noalloc call {i}")


def test_noalloc_refuses_oversized_plan(lib):
    import torch
    m, k, n = 168, 2560, 19456        # workspace 43.5 MB > 32 MiB of static scratch
    assert lib.gemm_workspace_size(m, n, k) > lib.STATIC_SCRATCH_BYTES
    x = torch.zeros((m, k), dtype=torch.float16, device="cuda")
    qw = torch.zeros((k // 8, n), dtype=torch.int32, device="cuda")
    sc = torch.zeros((k // 128, n), dtype=torch.float16, device="cuda")
    qz = torch.zeros((k // 128, n // 8), dtype=torch.int32, device="cuda")
    with pytest.raises(lib.W4VError):
        lib.w4a16_gemm_noalloc(x, qw, sc, qz)
