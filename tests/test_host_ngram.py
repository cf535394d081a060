"""The host prompt lookup of the generation driver (runner.ngram_lookup)
against the oracle's proposer, fixed lengths and windows, on random contexts
over a few ids (many repeats) and on short contexts."""
import numpy as np

from draft_then_verify_amd.runner import ngram_lookup
from oracle.ngram import ngram_propose, ngram_propose_window


def test_host_lookup_matches_oracle():
    rng = np.random.default_rng(21)
    for _ in range(600):
        L = int(rng.integers(0, 40))
        ctx = [int(t) for t in rng.integers(0, int(rng.integers(2, 6)), L)]
        n = int(rng.integers(1, 6))
        n_max = n + int(rng.integers(0, 6))
        g = int(rng.integers(0, 8))
        assert ngram_lookup(ctx, n, g) == ngram_propose(ctx, n, g)
        assert ngram_lookup(ctx, n, g, n_max) == ngram_propose_window(ctx, n, n_max, g)
