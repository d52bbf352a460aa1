"""Closed forms of the pages' speed-up model (test infrastructure).

[PT] "Decodificacao Especulativa e EAGLE-3", section "O que determina a
aceleracao" (and the Persian twin, "speed-up factors"): with a per-token
acceptance rate alpha and N drafts, the expected number of tokens produced by
one verifier pass is (1 - alpha^(N+1)) / (1 - alpha); the expected wall time
per produced token is (N*c + 1) / E[accepted], where c is the draft/verifier
cost ratio.  The speed-up over plain decoding is the reciprocal of that time.

These are pure functions of (alpha, c, N); they are pinned in
tests/test_oracle_analytic.py against the oracle's own Monte Carlo and
against the pages' worked numbers (with the discrepancies documented there).
"""
from __future__ import annotations

import math


def expected_tokens(alpha: float, n: int) -> float:
    """E[tokens per verifier pass] = 1 + alpha + ... + alpha^N."""
    if alpha == 1.0:
        return float(n + 1)
    return (1.0 - alpha ** (n + 1)) / (1.0 - alpha)


def time_per_token(alpha: float, c: float, n: int) -> float:
    """(N*c + 1) / E[accepted], in units of one verifier pass."""
    return (n * c + 1.0) / expected_tokens(alpha, n)


def speedup(alpha: float, c: float, n: int) -> float:
    return 1.0 / time_per_token(alpha, c, n)


def best_n(alpha: float, c: float, n_max: int = 200):
    """(N*, speed-up at N*) over N = 1..n_max."""
    best = max(range(1, n_max + 1), key=lambda n: speedup(alpha, c, n))
    return best, speedup(alpha, c, best)


def truncated_geometric_var(alpha: float, n: int) -> float:
    """Variance of tokens per pass, K+1, where P(K >= i) = alpha^i for i <= N."""
    # E[(K+1)^2] = sum_{j=0..N} (2j+1) P(K >= j)
    m1 = sum(alpha ** j for j in range(n + 1))
    m2 = sum((2 * j + 1) * alpha ** j for j in range(n + 1))
    return m2 - m1 * m1


def chi2_critical_95(df: int) -> float:
    from scipy.stats import chi2
    return float(chi2.ppf(0.95, df))


__all__ = ["expected_tokens", "time_per_token", "speedup", "best_n", "truncated_geometric_var",
           "chi2_critical_95", "math"]
