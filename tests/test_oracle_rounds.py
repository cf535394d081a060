"""Oracle round driver and n-gram proposer pins."""
import numpy as np

from oracle import model as OM
from oracle import rounds as R
from oracle.ngram import ngram_propose, ngram_propose_window
from synth import Shape, make_prompt, make_weights, round_uniforms

SHAPE = Shape("r", 64, 3, 4, 2, 16, 96, 64, "f32")


def _generate(draft_layers, gamma, n_new, seed=21, B=2, P=7):
    w = make_weights(SHAPE, seed=seed, norm="random", std=0.1)
    tgt = OM.Decoder(SHAPE, w)
    dft = OM.Decoder(SHAPE, w, n_layers=draft_layers)
    prompt = make_prompt(B, P, SHAPE.vocab, seed=seed)
    ct, cd = tgt.new_cache(B, P + n_new + gamma + 2), dft.new_cache(B, P + n_new + gamma + 2)
    R.prefill(tgt, ct, prompt)
    R.prefill(dft, cd, prompt)
    committed = [list(prompt[b]) for b in range(B)]
    rounds = []
    r = 0
    while min(len(c) for c in committed) < P + n_new:
        u = round_uniforms(seed, r, B, gamma)
        last = np.array([c[-1] for c in committed])
        prev = np.array([c[-2] for c in committed])
        xs, q = R.draft_round(dft, cd, prev, last, ct.length, gamma, u["u_draft"])
        out = R.verify_round(tgt, ct, last, xs, q, None, u["u_acc"], u["u_res"])
        for b in range(B):
            committed[b] += [int(t) for t in out["emitted"][b, :out["n"][b] + 1]]
        rounds.append((xs, q, out))
        r += 1
    return committed, rounds, ct, P


def test_round_loop_invariants():
    committed, rounds, ct, P = _generate(draft_layers=1, gamma=3, n_new=12)
    for xs, q, out in rounds:
        cnt = (out["emitted"] >= 0).sum(1)
        assert ((cnt >= 1) & (cnt <= 4)).all()
        for b in range(xs.shape[0]):
            assert (out["emitted"][b, :out["n"][b]] == xs[b, :out["n"][b]]).all()
    # the target cache holds every committed token except the last
    for b, c in enumerate(committed):
        assert ct.length[b] == len(c) - 1


def test_full_depth_draft_accepts_every_guess():
    """A drafter identical to the target proposes from q = p, so every guess
    passes and each round emits gamma + 1 tokens [P1 Algorithm 1 with
    p = q; P3 acceptance equals the shared mass]."""
    committed, rounds, ct, P = _generate(draft_layers=SHAPE.n_layers, gamma=3, n_new=10)
    for xs, q, out in rounds:
        assert np.abs(q - out["p"][:, :3]).max() < 1e-6
        assert (out["n"] == 3).all()


def test_speculative_output_is_plain_decoding_distribution():
    """Emitted tokens of the speculative loop follow the target's own
    distribution: over many seeds, the first generated token's histogram matches
    the target's p at the last prompt position (chi-square)."""
    from scipy import stats
    from oracle import sampler as S

    shape = Shape("r2", 32, 1, 2, 1, 16, 48, 8, "f32")
    w = make_weights(shape, seed=5, norm="random", std=0.3)
    tgt = OM.Decoder(shape, w)
    dft = OM.Decoder(shape.with_(n_layers=1), make_weights(shape, seed=6, std=0.3))
    B, P, g = 4000, 4, 2
    prompt = np.tile(make_prompt(1, P, shape.vocab, seed=5), (B, 1))
    ct, cd = tgt.new_cache(B, P + g + 2), dft.new_cache(B, P + g + 2)
    R.prefill(tgt, ct, prompt)
    R.prefill(dft, cd, prompt)
    u = round_uniforms(77, 0, B, g)
    xs, q = R.draft_round(dft, cd, prompt[:, -2], prompt[:, -1], ct.length, g, u["u_draft"])
    out = R.verify_round(tgt, ct, prompt[:, -1], xs, q, None, u["u_acc"], u["u_res"])
    p0 = out["p"][0, 0]
    obs = np.bincount(out["emitted"][:, 0], minlength=shape.vocab)
    assert stats.chisquare(obs, p0 / p0.sum() * B).pvalue > 1e-3
    # and the draft really differs from the target (acceptance below 1)
    assert out["n"].mean() < g


def test_ngram_proposer():
    ctx = [5, 6, 7, 8, 9, 1, 5, 6, 7]
    assert ngram_propose(ctx, 3, 4) == [8, 9, 1, 5]
    assert ngram_propose(ctx, 3, 2) == [8, 9]
    # the most recent earlier occurrence wins
    ctx2 = [1, 2, 3, 10, 1, 2, 3, 20, 21, 1, 2, 3]
    assert ngram_propose(ctx2, 3, 3) == [20, 21, 1]
    # proposals can run into the suffix itself and stop at the context end
    ctx3 = [4, 4, 4, 4]
    assert ngram_propose(ctx3, 3, 5) == [4]
    assert ngram_propose([1, 2, 3, 4], 3, 4) == []
    assert ngram_propose([1, 2, 3], 3, 4) == []
    assert ngram_propose(ctx, 3, 0) == []


def _window_brute(ctx, n_min, n_max, gamma):
    """Every (length, start) pair scored as (length, start): the largest wins."""
    L = len(ctx)
    best = None
    for n in range(n_min, n_max + 1):
        for s in range(0, L - n):
            if ctx[s:s + n] == ctx[L - n:]:
                best = max(best or (0, -1), (n, s))
    if best is None or gamma <= 0:
        return []
    n, s = best
    return ctx[s + n:s + n + gamma]


def test_ngram_window_prefers_the_longest_match():
    # the last 4 tokens occur once (start 0); the last 2 also later (start 6)
    ctx = [1, 2, 3, 4, 50, 51, 3, 4, 60, 61, 1, 2, 3, 4]
    assert ngram_propose_window(ctx, 2, 4, 3) == [50, 51, 3]
    assert ngram_propose(ctx, 2, 3) == [60, 61, 1]
    assert ngram_propose_window(ctx, 2, 2, 3) == [60, 61, 1]
    # no length in the window occurs earlier, but a shorter one does
    assert ngram_propose_window([9, 8, 7, 1, 2, 5, 2], 2, 3, 4) == []
    assert ngram_propose_window([9, 8, 7, 1, 2, 5, 2], 1, 3, 4) == [5, 2]
    # a window wider than the context falls through to the lengths that fit
    assert ngram_propose_window([7, 7], 1, 8, 3) == [7]


def test_ngram_window_brute_force():
    rng = np.random.default_rng(11)
    for _ in range(400):
        L = int(rng.integers(1, 30))
        ctx = [int(t) for t in rng.integers(0, 3, L)]
        n_min = int(rng.integers(1, 5))
        n_max = n_min + int(rng.integers(0, 5))
        g = int(rng.integers(0, 6))
        assert ngram_propose_window(ctx, n_min, n_max, g) == _window_brute(ctx, n_min, n_max, g)
        assert ngram_propose_window(ctx, n_min, n_min, g) == ngram_propose(ctx, n_min, g)


def test_greedy_speculation_reproduces_greedy_decoding():
    """At T = 0 speculative decoding is lossless token for token: the emitted
    sequence equals plain greedy decoding of the target [P3 "Exactness is a
    choice"], whatever the drafter proposes.  Plain greedy decoding here is
    one target forward per token and an argmax of its last row."""
    w = make_weights(SHAPE, seed=31, norm="random", std=0.1)
    B, P, n_new, gamma = 2, 6, 14, 3
    prompt = make_prompt(B, P, SHAPE.vocab, seed=31)
    tgt = OM.Decoder(SHAPE, w)
    cap = P + n_new + gamma + 2
    # plain greedy decoding
    cp = tgt.new_cache(B, cap)
    logits = tgt.forward(cp, prompt)
    cp.length = cp.length + P
    plain = [list(prompt[b]) for b in range(B)]
    for _ in range(n_new):
        nxt = logits[:, -1].argmax(-1)
        for b in range(B):
            plain[b].append(int(nxt[b]))
        logits = tgt.forward(cp, nxt[:, None])
        cp.length = cp.length + 1
    # speculative, greedy draft from a shallower model of the same weights
    for draft_layers in (1, 2):
        dft = OM.Decoder(SHAPE, w, n_layers=draft_layers)
        ct, cd = tgt.new_cache(B, cap), dft.new_cache(B, cap)
        R.prefill(tgt, ct, prompt)
        R.prefill(dft, cd, prompt)
        spec = [list(prompt[b]) for b in range(B)]
        accepted = 0
        r = 0
        while min(len(c) for c in spec) < P + n_new:
            u = round_uniforms(31, r, B, gamma)
            last = np.array([c[-1] for c in spec])
            prev = np.array([c[-2] for c in spec])
            xs, q = R.draft_round(dft, cd, prev, last, ct.length, gamma, u["u_draft"], temperature=0.0)
            assert set(np.unique(q)) <= {0.0, 1.0}
            out = R.verify_round(tgt, ct, last, xs, q, None, None, None, temperature=0.0)
            for b in range(B):
                spec[b] += [int(t) for t in out["emitted"][b, :out["n"][b] + 1]]
            accepted += int(out["n"].sum())
            r += 1
        for b in range(B):
            assert spec[b][:P + n_new] == plain[b]
        assert accepted > 0 and r < n_new  # the drafter's guesses were used
