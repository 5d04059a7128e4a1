"""The HBM read-bandwidth probe (a measurement helper): every 32-bit word of
the source is read exactly once, so the XOR of the per-block words equals the
XOR of the whole buffer computed on the host."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 48, (1 << 20) + 16, 64 << 20])
def test_reads_every_word_once(lib, nbytes):
    import torch
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    out = lib.read_probe(src)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(words))
