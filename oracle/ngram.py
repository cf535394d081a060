"""Oracle n-gram (prompt-lookup) proposer (test infrastructure).

The pages describe it as matching the recent context against earlier text and
copying what followed [P2 "The three proposers"; P1 "Checking it on a real
system", method "ngram"].  Reading taken for a fixed match length n: find the
most recent earlier occurrence of the last n context tokens and propose up to
gamma of the tokens that followed it.  No occurrence: no proposal.

The match length is a window [prompt_lookup_min, prompt_lookup_max]
[P2 "Dial It In", the knob table; "Experiment 2" runs it at 3..8]: a shorter
minimum matches more often but less reliably.  Reading taken: try the lengths
from the maximum down to the minimum and take the first (longest) that has an
earlier occurrence.
"""

from __future__ import annotations


def ngram_propose(context, n: int, gamma: int) -> list:
    """Up to gamma proposed tokens for the context (a sequence of ids)."""
    ctx = [int(t) for t in context]
    L = len(ctx)
    if gamma <= 0 or L < n + 1:
        return []
    key = ctx[L - n:]
    for start in range(L - n - 1, -1, -1):  # occurrences strictly before the suffix
        if ctx[start:start + n] == key:
            return ctx[start + n:start + n + gamma]
    return []


def ngram_propose_window(context, n_min: int, n_max: int, gamma: int) -> list:
    """The proposal of the longest match length in [n_min, n_max] that occurs
    earlier in the context; [] when none does."""
    for n in range(n_max, n_min - 1, -1):
        prop = ngram_propose(context, n, gamma)
        if prop:
            return prop
    return []
