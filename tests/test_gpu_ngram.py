"""The device n-gram (prompt-lookup) proposer against the oracle's: every
proposal and count bit-exact, on contexts split between a prefix row and the
tokens committed since, with planted repeats, Markov-chain prompts (many
matches), contexts shorter than n + 1, ragged lengths, the fill option and
match-length windows (longest length first)."""
import numpy as np
import pytest
import torch

from draft_then_verify_amd import binding as bd
from oracle.ngram import ngram_propose, ngram_propose_window
from synth import make_markov_table, markov_prompt

pytestmark = pytest.mark.gpu


def _device_propose(prefix_rows, prefix_len, out_rows, out_len, n, gamma, fill_off=None, n_max=None):
    B, P = prefix_rows.shape
    cap = out_rows.shape[1]
    dr = torch.full((B, max(gamma, 1)), 7, dtype=torch.int32, device="cuda")
    nd = torch.empty(B, dtype=torch.int32, device="cuda")
    nf = torch.empty(B, dtype=torch.int32, device="cuda")
    t = lambda a: None if a is None else torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    bd.spec_ngram_propose(B, n, n if n_max is None else n_max, gamma, t(prefix_rows), t(prefix_len), P, t(out_rows) if cap else None,
                          t(out_len) if cap else None, cap, t(fill_off), dr, nd, nf)
    torch.cuda.synchronize()
    return dr.cpu().numpy()[:, :gamma], nd.cpu().numpy(), nf.cpu().numpy()


def _check(prefix_rows, prefix_len, out_rows, out_len, n, gamma, fill_off=None, n_max=None):
    drafts, nd, nf = _device_propose(prefix_rows, prefix_len, out_rows, out_len, n, gamma, fill_off, n_max)
    B, P = prefix_rows.shape
    cap = out_rows.shape[1]
    for b in range(B):
        lp = P if prefix_len is None else int(prefix_len[b])
        lo = min(int(out_len[b]), cap) if cap else 0
        ctx = list(prefix_rows[b, :lp]) + list(out_rows[b, :lo])
        want = ngram_propose(ctx, n, gamma) if n_max is None else ngram_propose_window(ctx, n, n_max, gamma)
        assert nf[b] == len(want), (b, nf[b], want)
        if fill_off is not None:
            pad = [int(prefix_rows[b, min(max(fill_off[b] + i, 0), P - 1)]) for i in range(gamma - len(want))]
            want = want + pad
        assert nd[b] == len(want)
        assert list(drafts[b, :len(want)]) == want, (b, list(drafts[b]), want)
        assert (drafts[b, len(want):] == -1).all()
    return nf


@pytest.mark.parametrize("n,gamma", [(3, 10), (1, 4), (2, 7), (4, 3), (3, 1)])
def test_ngram_matches_oracle(n, gamma):
    """Contexts over 3 ids (most sequences find a match, often near the end)
    and order-2 Markov prompts over 512 ids (the copy-heavy workload's
    prompts: a pair of ids rarely recurs within a few hundred tokens), split
    at ragged points between the prefix row and the committed tokens."""
    B, P, cap = 40, 300, 64
    rng = np.random.default_rng(n * 100 + gamma)
    prefix = rng.integers(0, 3, size=(B, P)).astype(np.int32)
    out = rng.integers(0, 3, size=(B, cap)).astype(np.int32)
    out_len = rng.integers(0, cap + 5, size=B)  # some past cap (counted, not stored)
    prefix_len = rng.integers(n, P + 1, size=B)
    nf = _check(prefix, prefix_len, out, out_len, n, gamma)
    assert (nf > 0).sum() > B // 2
    table = make_markov_table(seed=50 + n)
    prefix = markov_prompt(B, P, table, seed=60 + gamma).astype(np.int32)
    out = markov_prompt(B, cap, table, seed=70 + n).astype(np.int32)
    _check(prefix, prefix_len, out, out_len, n, gamma)


def test_ngram_planted_and_edge_cases():
    """Hand-made rows: the most recent occurrence wins, proposals stop at the
    end of the context and may run into the suffix, short contexts and
    contexts without a repeat propose nothing."""
    P, cap = 12, 6
    rows = [
        ([1, 2, 3, 10, 1, 2, 3, 20, 21, 1, 2, 3], 12, [], 0),   # most recent earlier occurrence: [20, 21, 1, ...]
        ([4, 4, 4, 4, 0, 0, 0, 0, 0, 0, 0, 0], 4, [], 0),       # overlap with the suffix: [4]
        ([1, 2, 3, 4, 0, 0, 0, 0, 0, 0, 0, 0], 4, [], 0),       # no repeat
        ([1, 2, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0], 2, [3], 1),       # three tokens: shorter than n + 1
        ([5, 6, 7, 8, 9, 0, 0, 0, 0, 0, 0, 0], 5, [1, 5, 6, 7], 4),  # match spans prefix and committed tokens
        ([9, 9, 9, 9, 9, 9, 9, 9, 9, 9, 9, 9], 12, [9, 9, 9], 3),
    ]
    B = len(rows)
    prefix = np.array([r[0] for r in rows], np.int32)
    plen = np.array([r[1] for r in rows], np.int32)
    out = np.zeros((B, cap), np.int32)
    for b, r in enumerate(rows):
        out[b, :len(r[2])] = r[2]
    olen = np.array([r[3] for r in rows], np.int32)
    for gamma in (0, 1, 3, 5):
        _check(prefix, plen, out, olen, 3, gamma)
    # no committed tokens at all (cap 0)
    _check(prefix, plen, np.zeros((B, 0), np.int32), np.zeros(B, np.int32), 3, 4)


@pytest.mark.parametrize("B", [1, 64])
def test_ngram_fill_pads_to_gamma(B):
    """With fill offsets every sequence proposes gamma tokens: the lookup's,
    then the prefix from the offset."""
    P, cap, g = 200, 16, 10
    table = make_markov_table(seed=81)
    prefix = markov_prompt(B, P, table, seed=82).astype(np.int32)
    rng = np.random.default_rng(83)
    prefix[: B // 2] = rng.integers(0, 100000, size=(B // 2, P))  # random rows: mostly misses
    out = rng.integers(0, 512, size=(B, cap)).astype(np.int32)
    olen = rng.integers(0, cap + 1, size=B)
    off = rng.integers(0, P - g - 1, size=B)
    _check(prefix, None, out, olen, 3, g, fill_off=off)


@pytest.mark.parametrize("n_min,n_max,gamma", [(3, 8, 4), (1, 4, 10), (2, 16, 7), (5, 5, 3)])
def test_ngram_window_matches_oracle(n_min, n_max, gamma):
    """Match-length windows: contexts over 3 ids (long repeats, so the longest
    length usually wins), over 6 ids (the lengths in the window fall through
    to shorter ones) and Markov prompts, split at ragged points; plus rows
    whose last n_max tokens repeat once far back while a shorter suffix
    repeats recently."""
    B, P, cap = 48, 256, 48
    rng = np.random.default_rng(1000 + 10 * n_min + n_max)
    out_len = rng.integers(0, cap + 5, size=B)
    prefix_len = rng.integers(1, P + 1, size=B)
    for ids in (3, 6):
        prefix = rng.integers(0, ids, size=(B, P)).astype(np.int32)
        out = rng.integers(0, ids, size=(B, cap)).astype(np.int32)
        _check(prefix, prefix_len, out, out_len, n_min, gamma, n_max=n_max)
    table = make_markov_table(seed=90 + n_max)
    prefix = markov_prompt(B, P, table, seed=91).astype(np.int32)
    out = markov_prompt(B, cap, table, seed=92).astype(np.int32)
    _check(prefix, prefix_len, out, out_len, n_min, gamma, n_max=n_max)
    # planted: the last n_max tokens occur at the start, their last n_min
    # tokens also just before the end
    prefix = rng.integers(100, 200, size=(B, P)).astype(np.int32)
    tail = rng.integers(200, 300, size=(B, n_max)).astype(np.int32)
    prefix[:, :n_max] = tail
    prefix[:, P - n_max:] = tail
    prefix[:, P - n_max - 10:P - n_max - 10 + n_min] = tail[:, n_max - n_min:]
    nf = _check(prefix, None, np.zeros((B, 0), np.int32), np.zeros(B, np.int32), n_min, gamma, n_max=n_max)
    assert (nf > 0).all()
