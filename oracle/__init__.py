"""CPU oracle for speculative (draft-then-verify) decoding -- TEST INFRASTRUCTURE.

A plain, slow, deliberately unoptimised NumPy implementation of what the verify
hot path computes, written from the pages' description of the method:

* ``model``     the Llama-style target/draft forward pass (fp64 arithmetic; the
                bf16 rounding points of the precision contract are explicit);
* ``sampler``   softmax, the min(1, p/q) accept test, prefix truncation, the
                norm(max(0, p - q)) residual, the bonus token and the
                fixed-point inverse-CDF draw;
* ``rounds``    one speculative round and the drafter loops, teacher-forced;
* ``ngram``     the prompt-lookup (n-gram) proposer;
* ``economics`` the pages' closed forms (expected tokens per round, speedup
                models, break-even, the wall-clock division, the log metrics).

Only the test suite, the smoke entry point and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its Python
binding) never imports, calls or links anything here; the two share no code
apart from the seeded input generators in ``synth``.

Sources (the pages, by title):
  [P1] "Speculative Decoding Spends Arithmetic You May Not Have"
  [P2] "05 · Speculative Decoding"
  [P3] "How Speculative Decoding Works (and When It Doesn't)"
  [P4] "speculative-decoding-verify-cost" (the wall-clock division page)
  [P5] "Speculative Decoding Is a Bet on How Predictable Your Traffic Is"

Parity status: the forward pass has no printed logits on the pages; it is
pinned by invariants and by library special cases (see tests), not by page
values.
"""
