"""Oracle round drivers (test infrastructure; see package docstring).

One speculative round [P1 Algorithm 1; P5 "What it looks like in code"]:
draft gamma tokens autoregressively from the drafter, score [last committed,
x_1 .. x_gamma] with one target pass, run the sampler, commit.  Conventions:

* KV bookkeeping: the target cache holds every committed token except the
  last one; a round writes gamma + 1 rows and keeps n + 1 of them (the last
  committed token and the n accepted drafts).  The emitted token t becomes the
  new last committed token.
* A model drafter keeps its own cache.  Each round it re-feeds the last two
  committed tokens at positions L-1, L (its length is first set to L-1), so
  its first pass always has two rows; q_1 is the last row's softmax.
* The drafter samples x_i ~ q_i with the same fixed-point draw as the bonus.
* Teacher forcing: a caller checking another implementation passes that
  implementation's drafts (and q rows) in, so a mismatch never compounds.
"""

from __future__ import annotations

import numpy as np

from . import sampler


def verify_round(target, cache, last_tok, drafts, q, n_draft, u_acc, u_res, temperature=1.0):
    """Score, accept/resample and commit one round on the oracle's own target.
    temperature 0 verifies greedily (``sampler.greedy_verify``); q and the
    uniforms are then unused.

    Returns dict(logits fp64 [B, g+1, V], p fp64, n [B], emitted [B, g+1]).
    """
    last_tok = np.asarray(last_tok, np.int64).reshape(-1)
    B = last_tok.shape[0]
    drafts = np.asarray(drafts, np.int64).reshape(B, -1)
    tokens = np.concatenate([last_tok[:, None], drafts], axis=1)
    logits = target.forward(cache, tokens)
    p = sampler.softmax(logits, temperature)
    if float(temperature) == 0.0:
        n, emitted = sampler.greedy_verify(logits, drafts, n_draft)
    else:
        n, emitted = sampler.reject_sample(p.astype(np.float32), q, drafts, n_draft, u_acc, u_res)
    cache.length = cache.length + n + 1
    return {"logits": logits, "p": p, "n": n, "emitted": emitted}


def draft_round(draft, dcache, prev_tok, last_tok, target_len, gamma, u_draft, temperature=1.0):
    """gamma autoregressive draft steps.  Returns (drafts [B, g] int64, q [B, g, V] float32)."""
    prev_tok = np.asarray(prev_tok, np.int64).reshape(-1)
    last_tok = np.asarray(last_tok, np.int64).reshape(-1)
    dcache.length = np.asarray(target_len, np.int64) - 1
    inp = np.stack([prev_tok, last_tok], axis=1)
    xs, qs = [], []
    for i in range(gamma):
        logits = draft.forward(dcache, inp)
        dcache.length = dcache.length + inp.shape[1]
        qi = sampler.softmax(logits[:, -1], temperature).astype(np.float32)
        xi = sampler.sample(qi, np.asarray(u_draft, np.float32)[:, i])
        xs.append(xi)
        qs.append(qi)
        inp = xi[:, None]
    return np.stack(xs, axis=1), np.stack(qs, axis=1)


def prefill(model, cache, prompt):
    """Write K/V for prompt[:, :-1]; the last prompt token is the first round's input."""
    prompt = np.asarray(prompt, np.int64)
    if prompt.shape[1] > 1:
        model.forward(cache, prompt[:, :-1], logits=False)
        cache.length = cache.length + prompt.shape[1] - 1
