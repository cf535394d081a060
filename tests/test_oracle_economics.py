"""Oracle closed forms pinned to the numbers the pages print."""
import math

import pytest

from oracle import economics as ec
from tests._golden import load


def test_expected_tokens_p1():
    g = load("p1_expected_tokens.json")
    a = g["alpha"]
    for case in g["cases"]:
        assert round(ec.expected_tokens(a, case["gamma"]), 2) == case["tokens"]
    assert ec.expected_tokens_limit(a) == g["ceiling"]
    # closed form of the page equals the sum definition
    for gam in range(0, 20):
        assert math.isclose(ec.expected_tokens(a, gam), (1 - a ** (gam + 1)) / (1 - a), rel_tol=1e-12)
    assert round(1 / a ** 17) == g["gamma17_survival_one_in"]
    gain = ec.expected_tokens(a, 10) / ec.expected_tokens(a, 4) - 1
    assert round(100 * gain) == g["gain_gamma4_to_10_pct"]


def test_theorem_311_p1():
    g = load("p1_theorem311.json")
    assert round(ec.arithmetic_increase(g["alpha"], g["gamma"], g["c_hat"]), 2) == g["increase"]
    # the flattened exponent read the other way ((1-a^g)+1) does not reproduce the page
    a, gam = g["alpha"], g["gamma"]
    wrong = (1 - a) * (gam + 1) / (1 - a ** gam + 1)
    assert round(wrong, 2) != g["increase"]


def test_speedup_table_p2():
    g = load("p2_speedup_c010.json")
    for a_s, row in g["rows"].items():
        for k, v in zip(g["ks"], row):
            assert abs(ec.speedup_model(float(a_s), k, g["c"]) - v) <= 0.005 + 1e-9, (a_s, k)


def test_break_even_p2():
    g = load("p2_break_even.json")
    for k, v in g["bisection_c010"].items():
        assert f"{ec.break_even_alpha(int(k), 0.10):.3f}" == f"{v:.3f}"
    for c, row in g["table"].items():
        for k, v in row.items():
            assert abs(ec.break_even_alpha(int(k), float(c)) - v) <= 0.005 + 1e-9, (c, k)
    # a free proposer never loses
    for k in (2, 4, 8):
        assert ec.speedup_model(0.0, k, 0.0) >= 1.0
    for e in g["optimal_k_c010"]:
        k, s = ec.best_k(e["alpha"], 0.10)
        assert k == e["k"] and round(s, 2) == e["speedup"]
    assert round(ec.speedup_model(0.2, 8, 0.10), 2) == g["slowdown_alpha02_k8"]


def test_wallclock_division_p4():
    g = load("p4_division.json")
    assert round(1000.0 / g["plain_tok_s"], 2) == g["t_decode_ms"]
    tok_s = ec.wallclock_tok_per_s(g["p"], g["t_verify_ms"], g["t_draft_ms"])
    assert round(tok_s) == g["predicted_tok_s"]
    assert abs(tok_s / g["measured_tok_s"] - 1) < g["within_pct"] / 100
    # the ratio form equals tokens/s over plain tokens/s
    sp = ec.wallclock_speedup(g["p"], g["t_decode_ms"], g["t_verify_ms"], g["t_draft_ms"])
    assert math.isclose(sp, tok_s / (1000.0 / g["t_decode_ms"]), rel_tol=1e-12)
    be = ec.break_even_verify(g["p"], g["t_decode_ms"], g["t_draft_ms"])
    assert round(be, 1) == g["break_even_verify_ms"]
    assert round(be / g["t_decode_ms"], 2) == g["break_even_over_decode"]
    assert math.isclose(ec.wallclock_speedup(g["p"], g["t_decode_ms"], be, g["t_draft_ms"]), 1.0, rel_tol=1e-12)
    j = g["july"]
    wrong = ec.wallclock_tok_per_s(j["p"], 2 * j["block_sum_ms"], j["draft_ms"])
    right = ec.wallclock_tok_per_s(j["p"], 2 * j["graph_ms"], j["draft_ms"])
    assert round(wrong, 1) == j["wrong_tok_s"] and round(right, 1) == j["right_tok_s"]
    # the page's ratios mix rounded and unrounded tokens/s; both agree to 1e-3
    assert abs(wrong / j["graph_tok_s"] - j["wrong_ratio"]) < 1e-3
    assert abs(right / j["graph_tok_s"] - j["right_ratio"]) < 1e-3
    # corollary: verify = two decode passes loses for every p <= 1
    for p in (0.0, 0.5, 0.9, 1.0):
        assert ec.wallclock_speedup(p, 10.0, 20.0, 0.643) < 1.0
    assert round(ec.wallclock_speedup(1.0, j["graph_ms"], 2 * j["graph_ms"], j["draft_ms"]), 3) == j["p1_ceiling_ratio"]
    assert round(j["graph_ms"] - j["block_sum_ms"], 3) == j["missed_ms"]
    assert round(100 * (j["graph_ms"] - j["block_sum_ms"]) / j["block_sum_ms"], 1) == j["missed_pct"]


def test_log_metrics_p1():
    g = load("p1_spec_metrics.json")
    num_drafts = g["drafted"] // g["gamma"]
    assert round(100 * ec.acceptance_rate(g["accepted"], g["drafted"]), 1) == g["avg_draft_acceptance_pct"]
    mal = ec.mean_acceptance_length(g["accepted"], num_drafts)
    assert round(mal, 2) == g["mean_acceptance_length"]
    assert round(g["accepted_throughput"] / g["drafted_throughput"] * 100, 1) == g["avg_draft_acceptance_pct"]
    # per-position entries are unconditional, so they sum to MAL - 1
    assert abs(sum(g["per_position"]) - (mal - 1)) < 0.005
    # and they re-create the accepted count to within the printed rounding
    counts = [r * num_drafts for r in g["per_position"]]
    assert abs(sum(counts) - g["accepted"]) < 0.0005 * 4 * num_drafts
    rates = ec.per_position_rates(counts, num_drafts)
    assert rates == pytest.approx(g["per_position"])
