"""Prompt-lookup (n-gram) drafting and appending accepted tokens (oracle;
test infrastructure only).

Results page, section 3 (Table 3, drafting families, and the paragraph on
n-gram drafting): the n-gram / prompt-lookup drafter needs no auxiliary model
and copies spans from the prompt, at a K fixed per submission (K = 23 for the
team that used it); the drafts then go through the greedy verify, and the
accepted tokens extend the sequence.

Readings (the pages name the method and its K, nothing finer):
  * the drafter looks for an earlier occurrence of the last n tokens of the
    sequence's history, for n from n_max down to n_min, and uses the longest
    n that has one;
  * among the occurrences of that n it takes the most recent one; an
    occurrence must be followed by at least one token of the history, so it
    ends at a position e <= L - 2 (it may overlap the suffix itself);
  * the drafts are the up-to-K tokens that followed the occurrence; fewer
    than K (the span runs into the end of the history, or nothing matched)
    are padded with -1 sentinels to a constant K -- the padding the same
    section describes for constant-K drafts, lossless because a -1 is never
    accepted;
  * appending: the verify emits the accepted drafts plus the target's own
    next token, out_tokens[b][0 .. a_b]; those a_b + 1 tokens are appended to
    the history, as many as its capacity leaves room for.
Plain Python loops: for the small histories of the tests.
"""


def prompt_lookup(history, n_max: int, n_min: int, k: int):
    """Drafts for one history.  Returns (drafts [k] with -1 padding, n, e): the
    matched length and the end position of the occurrence (0, -1: no match)."""
    h = [int(t) for t in history]
    length = len(h)
    drafts = [-1] * k
    for n in range(n_max, n_min - 1, -1):
        if n > length - 1:             # no room for an earlier occurrence of n tokens
            continue
        suffix = h[length - n:]
        for e in range(length - 2, n - 2, -1):      # most recent first
            if h[e - n + 1:e + 1] == suffix:
                span = h[e + 1:e + 1 + k]
                drafts[:len(span)] = span
                return drafts, n, e
    return drafts, 0, -1


def prompt_lookup_batch(histories, n_max: int, n_min: int, k: int):
    """Drafts [B][k] for a list of histories (lists of token ids)."""
    return [prompt_lookup(h, n_max, n_min, k)[0] for h in histories]


def append_accepted(histories, capacity: int, out_tokens, accepted_len):
    """New histories: history b extended by out_tokens[b][0 .. accepted_len[b]]
    (a_b + 1 tokens), cut at `capacity` tokens."""
    result = []
    for h, out, a in zip(histories, out_tokens, accepted_len):
        new = [int(t) for t in h] + [int(t) for t in list(out)[:int(a) + 1]]
        result.append(new[:capacity])
    return result
