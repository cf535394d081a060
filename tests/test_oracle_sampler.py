"""Pins of the oracle's rejection sampler against what the pages and the
mathematics fix: the emitted distribution equals p [P1 "What one iteration
actually does"; P3 "Why the output doesn't change"], acceptance equals the
shared mass, the truncated-geometric length law [P1 "Why gamma has a
ceiling"], and the special cases (p = q, one-hot q, T -> 0)."""
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

from oracle import sampler as S
from synth import make_uniforms

SEED = 424242


def chisq_p(obs, probs):
    pr = np.asarray(probs, np.float64)
    pr = pr / pr.sum()
    return stats.chisquare(obs, pr * obs.sum()).pvalue


def dirichlet_rows(rng, n, V, alpha=1.0):
    return rng.dirichlet(np.full(V, alpha), size=n).astype(np.float32)


def test_fixed_point_draw_basics():
    V = 7
    # one-hot row always draws its index
    for i in range(V):
        r = np.zeros((3, V), np.float32)
        r[:, i] = 0.37
        t = S.fixed_point_draw(r, np.array([0.0, 0.5, 1 - 2 ** -24], np.float32))
        assert (t == i).all()
    # zero-mass entries are never drawn, lowest index wins at u = 0
    r = np.array([[0, 0, 0.25, 0, 0.75, 0, 0]], np.float32)
    assert S.fixed_point_draw(r, np.array([0.0], np.float32))[0] == 2
    u = make_uniforms((20000,), SEED, 99)
    t = S.fixed_point_draw(np.repeat(r, 20000, 0), u)
    assert set(np.unique(t)) <= {2, 4}
    # uniform row on V = 2**k entries: the draw is floor(u * V) exactly
    r = np.full((1, 8), 0.125, np.float32)
    uu = np.array([0, 0.124, 0.125, 0.5, 0.874, 0.875, 1 - 2 ** -24], np.float32)
    assert list(S.fixed_point_draw(np.repeat(r, len(uu), 0), uu)) == [0, 0, 1, 4, 6, 7, 7]
    # unnormalised rows are normalised by their sum
    r2 = np.array([[1.0, 1.0, 2.0]], np.float32) / np.float32(8)
    assert list(S.fixed_point_draw(np.repeat(r2, 4, 0), np.array([0.0, 0.26, 0.5, 0.76], np.float32))) == [0, 1, 2, 2]


def _round(p, q, x_draft, u_acc, u_res, n_draft=None):
    return S.reject_sample(p, q, x_draft, n_draft, u_acc, u_res)


def test_chi_square_emitted_equals_p_v8():
    """10**6 seeded rounds on V = 8: the first emitted token is distributed as
    p_1, and the bonus (all accepted) as p_{gamma+1}."""
    N, V, g = 10 ** 6, 8, 1
    rng = np.random.default_rng(SEED)
    p_rows = dirichlet_rows(rng, g + 1, V)
    q_rows = dirichlet_rows(rng, g, V)
    u_draft = make_uniforms((N,), SEED, 1)
    x = S.fixed_point_draw(np.broadcast_to(q_rows[0], (N, V)), u_draft)
    p = np.broadcast_to(p_rows, (N, g + 1, V))
    q = np.broadcast_to(q_rows, (N, g, V))
    n, em = _round(p, q, x[:, None], make_uniforms((N, g), SEED, 2), make_uniforms((N,), SEED, 3))
    obs = np.bincount(em[:, 0], minlength=V)
    assert chisq_p(obs, p_rows[0]) > 1e-3
    acc = n == g
    obs2 = np.bincount(em[acc, g], minlength=V)
    assert chisq_p(obs2, p_rows[g]) > 1e-3
    # acceptance probability = shared mass sum(min(p, q)) [P3]
    beta = np.minimum(p_rows[0], q_rows[0]).astype(np.float64).sum()
    assert abs(acc.mean() - beta) < 5 * np.sqrt(beta * (1 - beta) / N)


def test_chi_square_gamma4_first_token():
    N, V, g = 400_000, 8, 4
    rng = np.random.default_rng(SEED + 1)
    p_rows = dirichlet_rows(rng, g + 1, V)
    q_rows = dirichlet_rows(rng, g, V)
    xs = np.stack([S.fixed_point_draw(np.broadcast_to(q_rows[i], (N, V)), make_uniforms((N,), SEED, 10 + i))
                   for i in range(g)], 1)
    n, em = _round(np.broadcast_to(p_rows, (N, g + 1, V)), np.broadcast_to(q_rows, (N, g, V)), xs,
                   make_uniforms((N, g), SEED, 20), make_uniforms((N,), SEED, 21))
    obs = np.bincount(em[:, 0], minlength=V)
    assert chisq_p(obs, p_rows[0]) > 1e-3
    # second emitted token given the first draft was accepted is distributed as p_2
    m = n >= 1
    obs = np.bincount(em[m, 1], minlength=V)
    assert chisq_p(obs, p_rows[1]) > 1e-3


def _grid_counts(fn, V):
    """Exact outcome counts of fn over all 2**24 grid uniforms u = k / 2**24.

    fn maps a float32 array of uniforms to integer outcomes that are
    non-decreasing in u (true of the inverse-CDF draw and of the reject flag).
    The step boundaries are found by bisection, then the whole step function is
    checked against fn on a strided subset of the grid."""
    two24 = 1 << 24

    def f(k):
        return int(fn(np.array([k / two24], np.float32))[0])

    counts = np.zeros(V, np.int64)
    starts, labels = [], []
    lo, cur = 0, f(0)
    while True:
        starts.append(lo)
        labels.append(cur)
        a, b = lo, two24 - 1
        if f(b) == cur:
            counts[cur] += b - lo + 1
            break
        while b - a > 1:  # f(a) == cur < f(b)
            mid = (a + b) // 2
            if f(mid) == cur:
                a = mid
            else:
                b = mid
        counts[cur] += a - lo + 1
        lo, cur = b, f(b)
    ks = np.arange(0, two24, 4099)
    got = fn((ks / two24).astype(np.float32))
    expect = np.asarray(labels)[np.searchsorted(np.asarray(starts), ks, side="right") - 1]
    assert (got == expect).all()
    return counts


@pytest.mark.parametrize("case", [0, 1, 2])
def test_exact_enumeration_emitted_law(case):
    """Count every uniform of the grid for the draft, the accept test and the
    resample: P(emit t) equals p(t) up to the grid resolution (a few 2**-24),
    and P(accept) equals sum(min(p, q))."""
    rng = np.random.default_rng(SEED + 10 + case)
    V = 3 + case % 2
    p1 = dirichlet_rows(rng, 1, V, 0.7)[0]
    q1 = dirichlet_rows(rng, 1, V, 0.7)[0]
    if case == 2:  # disjoint-ish supports
        V = 4
        p1 = np.array([0.5, 0.5, 0.0, 0.0], np.float32)
        q1 = np.array([0.0, 0.25, 0.25, 0.5], np.float32)
    p2 = dirichlet_rows(rng, 1, V)[0]
    two24 = 1 << 24
    pdraft = _grid_counts(lambda u: S.fixed_point_draw(np.broadcast_to(q1, (len(u), V)), u), V)
    assert pdraft.sum() == two24
    P_emit = [Fraction(0)] * V
    P_acc_total = Fraction(0)
    pq = np.stack([p1, p2])
    for x in range(V):
        if pdraft[x] == 0:
            continue
        px = Fraction(int(pdraft[x]), two24)

        def rounds(u_acc, u_res):
            N = max(len(u_acc), len(u_res))
            return _round(np.broadcast_to(pq, (N, 2, V)), np.broadcast_to(q1[None], (N, 1, V)),
                          np.full((N, 1), x), np.broadcast_to(u_acc, (N,))[:, None],
                          np.broadcast_to(u_res, (N,)))

        # rejected (1) is non-decreasing in u_acc
        rej = _grid_counts(lambda u: 1 - rounds(u, np.zeros(1, np.float32))[0], 2)[1]
        pa = Fraction(two24 - int(rej), two24)
        P_acc_total += px * pa
        P_emit[x] += px * pa
        if rej > 0:
            # the largest u_acc rejects; count the resample over the u_res grid
            u_rej = np.array([1 - 2 ** -24], np.float32)
            res = _grid_counts(lambda u: rounds(u_rej, u)[1][:, 0], V)
            for t in range(V):
                P_emit[t] += px * (1 - pa) * Fraction(int(res[t]), two24)
    pn = p1.astype(np.float64) / p1.astype(np.float64).sum()
    for t in range(V):
        assert abs(float(P_emit[t]) - pn[t]) < 8 * 2 ** -24, (t, float(P_emit[t]), pn[t])
    beta = np.minimum(p1, q1).astype(np.float64).sum()
    assert abs(float(P_acc_total) - beta) < 8 * 2 ** -24


def test_iid_length_law_p1():
    """Same (p, q) at every position with shared mass 0.75: n is truncated
    geometric and E[n + 1] = (1 - a^5)/(1 - a) = 3.05 at gamma = 4 [P1]."""
    V, g, N = 8, 4, 400_000
    p_row = np.array([0.5, 0.5, 0, 0, 0, 0, 0, 0], np.float32)
    q_row = np.array([0.5, 0.25, 0.25, 0, 0, 0, 0, 0], np.float32)
    a = float(np.minimum(p_row, q_row).sum())
    assert a == 0.75
    xs = np.stack([S.fixed_point_draw(np.broadcast_to(q_row, (N, V)), make_uniforms((N,), SEED, 30 + i))
                   for i in range(g)], 1)
    n, em = _round(np.broadcast_to(p_row, (N, g + 1, V)), np.broadcast_to(q_row, (N, g, V)), xs,
                   make_uniforms((N, g), SEED, 40), make_uniforms((N,), SEED, 41))
    law = np.array([a ** i * (1 - a) for i in range(g)] + [a ** g])
    obs = np.bincount(n, minlength=g + 1)
    assert chisq_p(obs, law) > 1e-3
    mean = (n + 1).mean()
    assert abs(mean - (1 - a ** (g + 1)) / (1 - a)) < 5 * (n + 1).std() / np.sqrt(N)
    assert round((1 - a ** (g + 1)) / (1 - a), 2) == 3.05


def test_round_invariants_and_truncation():
    rng = np.random.default_rng(SEED + 2)
    B, g, V = 2000, 5, 16
    p = rng.dirichlet(np.ones(V), size=(B, g + 1)).astype(np.float32)
    q = rng.dirichlet(np.ones(V), size=(B, g)).astype(np.float32)
    xs = rng.integers(0, V, size=(B, g))
    nd = rng.integers(0, g + 1, size=B)
    n, em = _round(p, q, xs, make_uniforms((B, g), SEED, 50), make_uniforms((B,), SEED, 51), nd)
    count = (em >= 0).sum(1)
    assert ((count >= 1) & (count <= g + 1)).all()
    assert (count == n + 1).all()
    assert (n <= nd).all()
    for b in range(B):
        assert (em[b, :n[b]] == xs[b, :n[b]]).all()
        assert (em[b, n[b] + 1:] == -1).all()
        # prefix truncation: position n was tested and failed unless all passed
        if n[b] < nd[b]:
            i = n[b]
            assert not (np.float32(make_uniforms((B, g), SEED, 50)[b, i]) * q[b, i, xs[b, i]] <= p[b, i, xs[b, i]])


def test_p_equals_q_accepts_everything():
    rng = np.random.default_rng(SEED + 3)
    B, g, V = 500, 4, 32
    q = rng.dirichlet(np.ones(V), size=(B, g)).astype(np.float32)
    p = np.concatenate([q, rng.dirichlet(np.ones(V), size=(B, 1)).astype(np.float32)], 1)
    xs = rng.integers(0, V, size=(B, g))
    n, em = _round(p, q, xs, make_uniforms((B, g), SEED, 60), make_uniforms((B,), SEED, 61))
    assert (n == g).all()
    assert ((em >= 0).sum(1) == g + 1).all()


def test_one_hot_q_accepts_with_probability_p_x():
    N, V = 400_000, 6
    p_row = np.array([0.05, 0.4, 0.2, 0.1, 0.15, 0.1], np.float32)
    for x in (1, 3):
        n, em = _round(np.broadcast_to(p_row, (N, 2, V)), None, np.full((N, 1), x),
                       make_uniforms((N, 1), SEED, 70 + x), make_uniforms((N,), SEED, 80 + x))
        rate = (n == 1).mean()
        assert abs(rate - p_row[x]) < 5 * np.sqrt(p_row[x] * (1 - p_row[x]) / N)
        # the residual of a one-hot q zeroes only x: a rejected round never emits x
        assert not (em[n == 0, 0] == x).any()
        # exact form of the decision: accept iff u <= p(x)
        u = make_uniforms((N, 1), SEED, 70 + x)[:, 0]
        assert ((n == 1) == (u <= p_row[x])).all()


def test_q_zero_accepts_and_all_reject_emits_one():
    V = 5
    p = np.array([[[0.0, 0.5, 0.5, 0, 0], [0.2, 0.2, 0.2, 0.2, 0.2]]], np.float32)
    # q(x) = 0: the division-free rule accepts
    q = np.array([[[0.0, 1.0, 0, 0, 0]]], np.float32)
    n, em = _round(p, q, np.array([[0]]), np.array([[0.9]], np.float32), np.array([0.3], np.float32))
    assert n[0] == 1 and em[0, 0] == 0
    # one-hot q at a token with p = 0: always exactly one token, never x
    N = 10000
    n, em = _round(np.broadcast_to(p, (N, 2, V)), None, np.zeros((N, 1), int),
                   make_uniforms((N, 1), SEED, 90), make_uniforms((N,), SEED, 91))
    assert (n == 0).all() and (em[:, 1] == -1).all() and set(np.unique(em[:, 0])) <= {1, 2}


def test_all_zero_residual_falls_back_to_p():
    p = np.array([[[0.5, 0.25, 0.25], [1 / 3, 1 / 3, 1 / 3]]], np.float32)
    q = np.array([[[0.5 + 2 ** -20, 0.25, 0.25]]], np.float32)
    u_acc = np.array([[1 - 2 ** -24]], np.float32)
    for u in (0.1, 0.6, 0.9):
        n, em = _round(p, q, np.array([[0]]), u_acc, np.array([u], np.float32))
        assert n[0] == 0
        assert em[0, 0] == S.fixed_point_draw(p[:, 0], np.array([u], np.float32))[0]


def test_temperature_zero_limit_is_argmax():
    """T -> 0 collapses p to its argmax: a draft is accepted iff it is the argmax
    and the emitted token is always the argmax [P3 "Exactness is a choice"]."""
    rng = np.random.default_rng(SEED + 4)
    B, g, V = 300, 3, 20
    logits = rng.normal(size=(B, g + 1, V))
    p = S.softmax(logits, temperature=1e-4).astype(np.float32)
    amax = logits.argmax(-1)
    xs = np.where(rng.random((B, g)) < 0.5, amax[:, :g], rng.integers(0, V, size=(B, g)))
    n, em = _round(p, None, xs, make_uniforms((B, g), SEED, 95), make_uniforms((B,), SEED, 96))
    for b in range(B):
        match = xs[b] == amax[b, :g]
        expect_n = g if match.all() else int(np.argmin(match))
        assert n[b] == expect_n
        assert (em[b, :n[b] + 1] == amax[b, :n[b] + 1]).all()


def test_softmax_matches_scipy():
    rng = np.random.default_rng(SEED + 5)
    x = rng.normal(size=(7, 50)) * 3
    from scipy.special import softmax as sp_softmax
    assert np.allclose(S.softmax(x), sp_softmax(x, axis=-1), rtol=1e-13, atol=1e-15)
    assert np.allclose(S.softmax(x, 0.5), sp_softmax(2 * x, axis=-1), rtol=1e-13, atol=1e-15)


# ---- greedy (T = 0) verification -------------------------------------------------

def test_greedy_verify_hand_worked():
    """Worked by hand from the definition: a_i = argmax row i (lowest index on
    ties); accept while x_i == a_i; emit the accepted drafts and a_n."""
    L = np.array([[[0, 5, 1, 2],      # a_0 = 1
                   [3, 3, 0, 1],      # tie at 0 and 1 -> a_1 = 0
                   [0, 0, 9, 9],      # tie at 2 and 3 -> a_2 = 2
                   [7, 0, 0, 8]]],    # a_3 = 3
                 np.float32)
    # all three drafts agree: n = 3, bonus a_3
    n, em = S.greedy_verify(L, np.array([[1, 0, 2]]))
    assert n.tolist() == [3] and em.tolist() == [[1, 0, 2, 3]]
    # the tie loser (index 1 on row 1) is rejected and replaced by a_1 = 0
    n, em = S.greedy_verify(L, np.array([[1, 1, 2]]))
    assert n.tolist() == [1] and em.tolist() == [[1, 0, -1, -1]]
    # first draft wrong: n = 0, emit a_0
    n, em = S.greedy_verify(L, np.array([[3, 0, 2]]))
    assert n.tolist() == [0] and em.tolist() == [[1, -1, -1, -1]]
    # ragged: only the first 2 drafts count, so the bonus comes from row 2
    n, em = S.greedy_verify(L, np.array([[1, 0, 3]]), n_draft=[2])
    assert n.tolist() == [2] and em.tolist() == [[1, 0, 2, -1]]
    # gamma = 0: the round is one greedy decoding step
    n, em = S.greedy_verify(L[:, :1], np.zeros((1, 0), np.int64))
    assert n.tolist() == [0] and em.tolist() == [[1]]


def test_greedy_ties_and_infinities():
    L = np.full((1, 1, 9000), -np.inf, np.float32)
    assert S.greedy_verify(L, np.zeros((1, 0)))[1].tolist() == [[0]]   # all -inf: lowest index
    L[0, 0, [4097, 8191, 8999]] = 2.5
    assert S.greedy_verify(L, np.zeros((1, 0)))[1].tolist() == [[4097]]
    L[0, 0, 12] = np.inf
    assert S.greedy_verify(L, np.zeros((1, 0)))[1].tolist() == [[12]]


def test_greedy_is_the_zero_temperature_limit_of_the_exact_rule():
    """[P3 "Exactness is a choice"]: at T -> 0 the exact rule and greedy pick
    the same tokens.  The exact rule (reject_sample) on softmax(l / 1e-4) with
    a one-hot draft must reproduce greedy_verify for any uniforms in (0, 1)."""
    rng = np.random.default_rng(SEED + 40)
    B, g, V = 400, 5, 33
    logits = rng.normal(size=(B, g + 1, V)) * 3
    a = logits.argmax(-1)
    xs = np.where(rng.random((B, g)) < 0.7, a[:, :g], rng.integers(0, V, size=(B, g)))
    nd = rng.integers(0, g + 1, size=B)
    n_g, em_g = S.greedy_verify(logits, xs, nd)
    p = S.softmax(logits, temperature=1e-4).astype(np.float32)
    for s in range(3):
        n_e, em_e = _round(p, None, xs, make_uniforms((B, g), SEED, 97, s), make_uniforms((B,), SEED, 98, s), nd)
        assert np.array_equal(n_g, n_e) and np.array_equal(em_g, em_e)
    assert 0 < n_g.mean() < g  # both outcomes occur


def test_softmax_temperature_zero_is_one_hot_at_argmax():
    L = np.array([[1.0, 3.0, 3.0, -2.0], [0.0, 0.0, 0.0, 0.0]])
    assert S.softmax(L, 0.0).tolist() == [[0, 1, 0, 0], [1, 0, 0, 0]]
    rng = np.random.default_rng(SEED + 41)
    x = rng.normal(size=(50, 17))
    assert np.array_equal(S.softmax(x, 0.0).argmax(-1), x.argmax(-1))
    assert np.allclose(S.softmax(x, 0.0), S.softmax(x, 1e-6), atol=1e-12)
