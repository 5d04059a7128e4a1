"""CPU oracle for the W4A16 speculative-verify path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 numpy definitions of what the verify step computes.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product path (the HIP library and its Python
binding) never does, and this package never imports the product path.  The
two sides share nothing but the seeded input module ``gen``.

Sources (organisers' page "Efficient LLM Challenge Results", adaptfm.gitlab.io):
  section 3  -- speculative decoding: one target pass checks K drafts,
                which are kept up to the first that differs from the target's
                greedy token; greedy serving; the winner's target is W4A16 GPTQ
                with group size 128 and an untied lm_head quantised to 8 bits;
                the runner-up fills drafts up to K=20 with -1, which never
                matches a vocabulary id.
                Table 3 and the paragraph on n-gram drafting: the prompt-
                lookup drafter copies spans from the prompt, no auxiliary
                model, fixed K (23 for the team that used it).
  section 5  -- W4A16 (group size 128), W8A16 lm_head; team #5's target:
                W4A16 with group size 32, the first two and last two layers
                and the lm_head in half precision.

Modules:
  quant   -- int4 unpacking and group dequantisation
  gemm    -- the W4A16 linear (group size 128 or 32), the fp16 linear, fp16
             storage rounding
  lmhead  -- 8-bit and fp16 lm_head logits, argmax with tie-break, top-2 margin
  verify  -- greedy prefix acceptance with sentinels, verified-token count
  step    -- the free-running verify step (chain of linears, lm_head, verify)
  ngram   -- prompt-lookup drafting and appending the accepted tokens
  gdn     -- committing a Gated DeltaNet state to the accepted prefix

Every function is pinned by a ``-m "not gpu"`` test (pack/unpack round trips,
hand-built words, identity and one-hot weights, closed forms, exact-rational
brute force on tiny shapes, exhaustive enumeration for the verify and the
drafter; the chain of ``step`` by permutation chains with mixed widths and
hand-worked rounding cases in ``tests/test_oracle_step.py``).
"""
from . import quant, gemm, lmhead, verify, step, ngram, gdn  # noqa: F401
