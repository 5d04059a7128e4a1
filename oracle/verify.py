"""Greedy prefix acceptance (oracle; test infrastructure only).

Results page, section 3: the target verifies K drafted tokens in one forward
pass and keeps the longest prefix it would itself have produced; under greedy
verification the output is unchanged whatever the drafts are.  Drafts padded
to a constant K with -1 sentinels stay lossless because a padded position is
accepted only when it equals the target's own greedy token -- which a -1
never does.

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
