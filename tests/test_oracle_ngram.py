"""Pins for the prompt-lookup drafting oracle: hand-worked golden cases, an
exhaustive search over all (n, e) pairs on tiny random histories, and the
span property of every proposal."""
import json
import os

import numpy as np

from oracle import ngram

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ngram_cases.json")))


def test_golden_drafts():
    for c in GOLDEN["draft_cases"]:
        d, n, e = ngram.prompt_lookup(c["history"], c["n_max"], c["n_min"], c["k"])
        assert d == c["drafts"], c["name"]
        assert (n, e) == (c["n"], c["e"]), c["name"]


def test_golden_append():
    for c in GOLDEN["append_cases"]:
        got = ngram.append_accepted(c["histories"], c["capacity"], c["out_tokens"], c["accepted_len"])
        assert got == c["result"], c["name"]


def _exhaustive(h, n_max, n_min):
    """Every (n, e) with h[e-n+1 .. e] equal to the last n tokens and e <= L-2;
    the answer is the lexicographically largest pair."""
    best = (0, -1)
    length = len(h)
    for n in range(n_min, n_max + 1):
        for e in range(n - 1, length - 1):
            if length - n >= 0 and all(h[e - i] == h[length - 1 - i] for i in range(n)):
                best = max(best, (n, e))
    return best


def test_exhaustive_tiny_histories():
    rng = np.random.default_rng(5)
    for trial in range(400):
        length = int(rng.integers(0, 24))
        vocab = int(rng.integers(2, 5))
        h = [int(t) for t in rng.integers(0, vocab, length)]
        n_min = int(rng.integers(1, 4))
        n_max = n_min + int(rng.integers(0, 4))
        k = int(rng.integers(1, 6))
        d, n, e = ngram.prompt_lookup(h, n_max, n_min, k)
        assert (n, e) == _exhaustive(h, n_max, n_min), (h, n_max, n_min)
        if n == 0:
            assert d == [-1] * k
        else:
            span = h[e + 1:e + 1 + k]
            assert d == span + [-1] * (k - len(span))
            # the occurrence ends where the drafted span starts, and equals the suffix
            assert h[e - n + 1:e + 1] == h[len(h) - n:]


def test_batch_matches_single():
    hs = [[1, 2, 1, 2], [3], [], [4, 5, 6, 4, 5]]
    assert ngram.prompt_lookup_batch(hs, 3, 1, 3) == [ngram.prompt_lookup(h, 3, 1, 3)[0] for h in hs]
