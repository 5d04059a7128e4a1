"""GPU parity of prompt-lookup drafting and of appending accepted tokens
against the oracle (exact integers), and a closed draft -> verify -> append
loop against the same loop on the CPU."""
import numpy as np
import pytest

import gen
from oracle import ngram, verify as ov
from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


def gpu_draft(lib, hist, lengths, n_max, n_min, k):
    import torch
    d = lib.ngram_draft(dev(hist), dev(np.asarray(lengths, np.int32)), n_max, n_min, k)
    torch.cuda.synchronize()
    return host(d)


def oracle_draft(hist, lengths, n_max, n_min, k):
    return np.asarray([ngram.prompt_lookup(list(hist[b, :lengths[b]]), n_max, n_min, k)[0]
                       for b in range(len(lengths))], dtype=np.int32)


@pytest.mark.parametrize("vocab", [4, 50, 151936])
@pytest.mark.parametrize("n_max,n_min,k", [(1, 1, 1), (3, 1, 15), (4, 2, 23), (8, 1, 20)])
def test_drafts_match_oracle(lib, vocab, n_max, n_min, k):
    rng = np.random.default_rng(vocab + 31 * n_max + 7 * k)
    lengths = [0, 1, 2, 3, 5, 64, 257, 300, 1000]
    cap = 1100
    hist = gen.token_histories(rng, lengths, cap, vocab)
    # garbage past each row's length: the drafter must not read it
    for b, n in enumerate(lengths):
        hist[b, n:] = rng.integers(0, vocab, cap - n)
    got = gpu_draft(lib, hist, lengths, n_max, n_min, k)
    ref = oracle_draft(hist, lengths, n_max, n_min, k)
    assert np.array_equal(got, ref)
    log(f"  vocab {vocab} n {n_min}..{n_max} K={k}: {int(np.sum(ref[:, 0] >= 0))}/{len(lengths)} matched")


def test_long_bucket_histories(lib):
    """8,192-token histories (the long prompt bucket), K = 23, n 1..4."""
    rng = np.random.default_rng(8192)
    lengths = [8192, 8191, 4097, 2048, 8000, 64, 8192, 7000]
    hist = gen.token_histories(rng, lengths, 8192, 1000)
    got = gpu_draft(lib, hist, lengths, 4, 1, 23)
    ref = oracle_draft(hist, lengths, 4, 1, 23)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("n_max,n_plant", [(4, 4), (4, 3), (64, 64), (64, 40)])
def test_multi_tile_histories(lib, n_max, n_plant):
    """Histories of 20,000+ tokens (the kernel stages 8,192 candidates at a time, newest
    first, with 64 tokens of look-back): the only long occurrence of the suffix is planted
    at the edges of the older tiles, where its earlier tokens sit in the look-back region,
    while a shorter occurrence sits in the newest tile."""
    rng = np.random.default_rng(20000 + n_max + n_plant)
    L = 20000
    ends = [L - 2 - 8192, L - 2 - 8191, L - 2 - 16383, L - 2 - 16384, L - 2 - 8192 - 60, n_plant - 1]
    cap = L + 37
    hist = rng.integers(0, 151936, (len(ends), cap)).astype(np.int32)
    for b, e in enumerate(ends):
        suffix = hist[b, L - n_plant:L].copy()
        hist[b, e - n_plant + 1:e + 1] = suffix
        # a shorter occurrence in the newest tile, which must lose to the planted one
        hist[b, L - 300 - 1:L - 300 + 1] = suffix[-2:]
    lengths = [L] * len(ends)
    got = gpu_draft(lib, hist, lengths, n_max, 1, 23)
    ref = oracle_draft(hist, lengths, n_max, 1, 23)
    assert np.array_equal(got, ref)
    for b, e in enumerate(ends):           # the planted occurrence is the one that wins
        assert ngram.prompt_lookup(list(hist[b, :L]), n_max, 1, 23)[1:] == (n_plant, e)
        assert got[b].tolist() == hist[b, e + 1:e + 24].tolist()


def test_long_history_many_tiles(lib):
    """Copy-heavy histories of up to 40,000 tokens over a small vocabulary, against the oracle."""
    rng = np.random.default_rng(40000)
    lengths = [40000, 33000, 16385, 8193, 24577]
    hist = gen.token_histories(rng, lengths, 40000, 3000)
    for n_max, n_min in [(4, 1), (12, 3), (64, 8)]:
        got = gpu_draft(lib, hist, lengths, n_max, n_min, 23)
        ref = oracle_draft(hist, lengths, n_max, n_min, 23)
        assert np.array_equal(got, ref), (n_max, n_min)


def test_golden_cases_on_gpu(lib):
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ngram_cases.json")))
    for c in g["draft_cases"]:
        h = np.full((1, max(1, len(c["history"]))), -1, np.int32)
        h[0, :len(c["history"])] = c["history"]
        got = gpu_draft(lib, h, [len(c["history"])], c["n_max"], c["n_min"], c["k"])
        assert got[0].tolist() == c["drafts"], c["name"]


def test_append_matches_oracle(lib):
    import torch
    rng = np.random.default_rng(3)
    B, K, cap = 6, 15, 40
    lengths = np.array([0, 5, 20, 38, 40, 25], np.int32)
    hist = gen.token_histories(rng, lengths, cap, 100)
    out = rng.integers(0, 100, (B, K + 1)).astype(np.int32)
    acc = np.array([0, 15, 3, 7, 2, 40], np.int32)            # the last is clamped to K
    h_d, l_d = dev(hist), dev(lengths)
    lib.append_accepted(h_d, l_d, dev(out), dev(acc))
    torch.cuda.synchronize()
    ref = ngram.append_accepted([list(hist[b, :lengths[b]]) for b in range(B)], cap, out,
                                np.minimum(acc, K))
    got_h, got_l = host(h_d), host(l_d)
    for b in range(B):
        assert got_l[b] == len(ref[b])
        assert got_h[b, :got_l[b]].tolist() == ref[b]
        assert np.array_equal(got_h[b, got_l[b]:], hist[b, got_l[b]:])   # untouched past the end


def test_closed_loop(lib):
    """Six rounds of draft (GPU) -> stand-in target ids -> greedy verify (GPU) -> append (GPU)
    for four sequences, against the same rounds through the oracle."""
    import torch
    rng = np.random.default_rng(77)
    B, K, V, cap = 4, 15, 64, 600
    lengths = np.array([120, 300, 64, 200], np.int32)
    hist = gen.token_histories(rng, lengths, cap, V)
    h_d, l_d = dev(hist), dev(lengths)
    cpu = [list(hist[b, :lengths[b]]) for b in range(B)]
    emitted = 0
    for r in range(6):
        d = lib.ngram_draft(h_d, l_d, 4, 1, K)
        torch.cuda.synchronize()
        gh, gl = host(h_d), host(l_d)
        # the GPU state equals the CPU state before every round
        assert [gh[b, :gl[b]].tolist() for b in range(B)] == cpu, r
        dd = host(d)
        ref_d = np.asarray(ngram.prompt_lookup_batch(cpu, 4, 1, K), np.int32)
        assert np.array_equal(dd, ref_d), r
        tgt = np.stack([gen.synthetic_target_ids(cpu[b], ref_d[b], V) for b in range(B)])
        acc_d, out_d = lib.greedy_verify(dev(tgt), d, V)
        lib.append_accepted(h_d, l_d, out_d, acc_d)
        acc_r, out_r = ov.greedy_verify(tgt, ref_d, V)
        assert np.array_equal(host(acc_d), acc_r.astype(np.int32)), r
        cpu = ngram.append_accepted(cpu, cap, out_r, acc_r)
        emitted += ov.verified_tokens(acc_r)
    torch.cuda.synchronize()
    gh, gl = host(h_d), host(l_d)
    assert [gh[b, :gl[b]].tolist() for b in range(B)] == cpu
    log(f"  closed loop: {emitted} tokens over 6 rounds x {B} sequences "
        f"({emitted / (6 * B):.2f} per verify)")
