"""Closed forms the pages state about the method (test infrastructure).

Each function is the definition as the page gives it, in plain Python floats.
"""

from __future__ import annotations


def expected_tokens(alpha: float, gamma: int) -> float:
    """Expected tokens committed per round under i.i.d. acceptance alpha with
    gamma drafts: position i (0 = the guaranteed token) is committed with
    probability alpha**i, so the sum runs over i = 0..gamma
    [P2 "The economics", expected tokens per step; P3 "Why the output doesn't
    change", expected committed tokens; P1 "Why gamma has a ceiling", the
    closed form (1 - alpha^(gamma+1)) / (1 - alpha)]."""
    return sum(alpha ** i for i in range(gamma + 1))


def expected_tokens_limit(alpha: float) -> float:
    """gamma -> infinity limit of expected_tokens: 1 / (1 - alpha) [P1 "Why gamma has a ceiling"]."""
    return 1.0 / (1.0 - alpha)


def speedup_model(alpha: float, k: int, c: float) -> float:
    """Tokens per step over cost per step, (sum_i alpha^i) / (1 + k c)
    [P2 "The economics -- one formula that decides everything"]."""
    return expected_tokens(alpha, k) / (1.0 + k * c)


def break_even_alpha(k: int, c: float, iters: int = 60) -> float:
    """Smallest alpha with speedup_model >= 1, by bisection on [0, 1]
    [P2 "The break-even is a real threshold you can compute"]."""
    lo, hi = 0.0, 1.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if speedup_model(mid, k, c) < 1.0:
            lo = mid
        else:
            hi = mid
    return lo


def best_k(alpha: float, c: float, ks=(1, 2, 3, 4, 6, 8)):
    """The k of largest speedup_model among ks, and that speedup [P2 "Cheat Sheet", optimal k]."""
    best = max(ks, key=lambda k: speedup_model(alpha, k, c))
    return best, speedup_model(alpha, best, c)


def arithmetic_increase(alpha: float, gamma: int, c_hat: float) -> float:
    """Expected increase in total arithmetic, Theorem 3.11 as quoted on
    [P1 "The speedup is borrowed"]: (1 - alpha)(gamma c_hat + gamma + 1) /
    (1 - alpha^(gamma + 1)).  The page's flattened exponent is read as
    alpha^(gamma+1), which is what reproduces its 1.64x."""
    return (1.0 - alpha) * (gamma * c_hat + gamma + 1) / (1.0 - alpha ** (gamma + 1))


def wallclock_speedup(p: float, t_decode: float, t_verify: float, t_draft: float) -> float:
    """(1 + p) T_decode / (T_verify + T_draft): tokens per round over time per
    round against plain decode, one draft per round [P4 "2. The division"]."""
    return (1.0 + p) * t_decode / (t_verify + t_draft)


def wallclock_tok_per_s(p: float, t_verify_ms: float, t_draft_ms: float) -> float:
    """Speculative throughput (1 + p) / (T_verify + T_draft), in tokens/s for times in ms [P4 "2. The division"]."""
    return (1.0 + p) / (t_verify_ms + t_draft_ms) * 1000.0


def break_even_verify(p: float, t_decode: float, t_draft: float) -> float:
    """Largest T_verify with wallclock_speedup >= 1: (1 + p) T_decode - T_draft [P4 "2.2 The break-even line"]."""
    return (1.0 + p) * t_decode - t_draft


# --- the engine's log metrics [P1 "Checking it on a real system"] -------------

def acceptance_rate(num_accepted: int, num_draft_tokens: int) -> float:
    """accepted tokens / drafted tokens."""
    return num_accepted / num_draft_tokens


def mean_acceptance_length(num_accepted: int, num_drafts: int) -> float:
    """1 + accepted tokens / number of drafts (rounds): the bonus token plus the accepted ones."""
    return 1.0 + num_accepted / num_drafts


def per_position_rates(accepted_per_pos, num_drafts: int):
    """Accepted count at each draft position over all drafts (unconditional)."""
    return [a / num_drafts for a in accepted_per_pos]
