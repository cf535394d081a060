"""Host-side acceptance statistics of the generation driver
(runner.acceptance_stats), pinned to definitions computed another way."""
import numpy as np
from scipy import optimize

from draft_then_verify_amd.runner import acceptance_stats, wilson_interval
from oracle import sampler as S


def test_per_position_sums_to_mal_minus_one():
    # the first page's log identity: the per-position acceptance rates add up
    # to the mean acceptance length minus one (section "Checking it on a real system")
    rng = np.random.default_rng(0)
    seqs = [rng.integers(0, 5, size=rng.integers(1, 40)) for _ in range(7)]
    st = acceptance_stats(seqs, 4)
    assert abs(sum(st["per_position"]) - (st["mean_acceptance_length"] - 1)) < 1e-12
    allv = np.concatenate(seqs)
    assert st["rounds_counted"] == allv.size
    assert abs(st["acceptance_rate"] - allv.sum() / (4 * allv.size)) < 1e-12


def test_wilson_interval_solves_its_inequality():
    # the Wilson interval is the set of p with |k/n - p| <= z sqrt(p (1 - p) / n);
    # find its ends by bisection
    for k, n in ((0, 10), (3, 10), (40, 100), (100, 100), (10312, 25600)):
        lo, hi = wilson_interval(k, n)
        ph, z = k / n, 1.96
        f = lambda p: (ph - p) ** 2 - z * z * p * (1 - p) / n
        # ph itself is inside (f(ph) <= 0); when ph sits at 0 or 1 (a root of
        # f there) start the search just inside
        inner = min(max(ph, 1e-12), 1 - 1e-12)
        lo_ref = 0.0 if f(0.0) <= 0 and ph == 0 else optimize.brentq(f, 0.0, inner)
        hi_ref = 1.0 if f(1.0) <= 0 and ph == 1 else optimize.brentq(f, inner, 1.0)
        assert abs(lo - lo_ref) < 1e-9 and abs(hi - hi_ref) < 1e-9


def test_geometric_fit_is_the_likelihood_maximum():
    rng = np.random.default_rng(1)
    g = 4
    ns = np.minimum(rng.geometric(0.35, size=500) - 1, g)
    st = acceptance_stats([ns], g)

    def nll(a):
        # P(n = k) = a^k (1 - a) for k < g, P(n = g) = a^g
        return -(np.log(a) * ns.sum() + np.log1p(-a) * (ns < g).sum())

    a_ref = optimize.minimize_scalar(nll, bounds=(1e-6, 1 - 1e-6), method="bounded",
                                     options={"xatol": 1e-10}).x
    assert abs(st["geometric_alpha"] - a_ref) < 1e-6
    assert abs(st["geometric_mal"] - sum(a_ref ** i for i in range(g + 1))) < 1e-5


def test_geometric_fit_recovers_alpha_from_the_oracle_law():
    # accepted lengths drawn by the oracle's own rule with i.i.d. acceptance
    # alpha = sum min(p, q) recover alpha (first page, "Why gamma has a ceiling")
    rng = np.random.default_rng(2)
    V, g, R = 6, 4, 4000
    p = np.array([0.3, 0.25, 0.2, 0.1, 0.1, 0.05], np.float32)
    q = np.array([0.1, 0.3, 0.2, 0.2, 0.1, 0.1], np.float32)
    alpha = float(np.minimum(p, q).sum())
    P = np.broadcast_to(p, (R, g + 1, V)).copy()
    Q = np.broadcast_to(q, (R, g, V)).copy()
    k = rng.integers(0, 1 << 24, size=(R, g)) / float(1 << 24)
    drafts = S.fixed_point_draw(np.broadcast_to(q, (R * g, V)), k.reshape(-1).astype(np.float32)).reshape(R, g)
    u_acc = (rng.integers(0, 1 << 24, size=(R, g)) / float(1 << 24)).astype(np.float32)
    u_res = (rng.integers(0, 1 << 24, size=R) / float(1 << 24)).astype(np.float32)
    n, _ = S.reject_sample(P, Q, drafts, None, u_acc, u_res)
    st = acceptance_stats([n], g)
    assert abs(st["geometric_alpha"] - alpha) < 0.02
    lo, hi = st["acceptance_rate_ci95"]
    assert lo < st["acceptance_rate"] < hi
