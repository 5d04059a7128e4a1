"""Greedy prefix acceptance (oracle; test infrastructure only).

Results page ("Efficient LLM Challenge Results", section 3): one forward pass
of the target checks all K drafts, and the drafts survive up to the first one
that differs from the target's own greedy choice at that position; with greedy
decoding this leaves the emitted text exactly what the target alone would
write.  The runner-up fills short drafts up to a fixed K with -1; since -1 is
no vocabulary id, a filler can never match, and the padding cannot change what
is accepted.

Row j of sequence b's target ids (j = 0..K) is the target's greedy token after
consuming the current token and drafts 0..j-1.  The accepted length a is the
number of leading drafts equal to their target token; the emitted tokens are
the accepted drafts plus the target's token at position a (the bonus), which
equals target[0..a].  Ids outside [0, V) -- the -1 sentinel among them --
never compare equal.
"""
import numpy as np


def greedy_verify(target_ids, draft_ids, vocab: int):
    """target_ids [B, K+1], draft_ids [B, K] -> (accepted_len [B], out_tokens [B, K+1]).

    out_tokens[b] = target_ids[b, 0..a_b] followed by -1.
    """
    t = np.asarray(target_ids, dtype=np.int64)
    d = np.asarray(draft_ids, dtype=np.int64)
    b_count, k1 = t.shape
    k = k1 - 1
    assert d.shape == (b_count, k)
    acc = np.zeros(b_count, dtype=np.int64)
    out = np.full((b_count, k1), -1, dtype=np.int64)
    for b in range(b_count):
        a = 0
        while a < k and 0 <= d[b, a] < vocab and d[b, a] == t[b, a]:
            a += 1
        acc[b] = a
        out[b, :a + 1] = t[b, :a + 1]
    return acc, out


def verified_tokens(accepted_len) -> int:
    """Tokens a verify step emits: sum over sequences of (a_b + 1)."""
    return int(np.sum(np.asarray(accepted_len, dtype=np.int64) + 1))
