"""The pages' speed-up model checked against its own printed formula.

[PT] "Decodificacao Especulativa e EAGLE-3" (ai-engineering.academy),
section "O que determina a aceleracao", Implementando Passo 6 and
Exercicios 2; [ZH] "投机解码与 EAGLE" section 2 ("when does it speed up":
the break-even alpha > c).  The formula values are asserted; where a worked
number the pages print does not follow from the formula, the test records
that instead of bending the formula.
"""
import pytest

from oracle import analytic as A


def test_expected_tokens_edge_values():
    """E = 1 at alpha = 0, N + 1 at alpha = 1, and the geometric sum between."""
    assert A.expected_tokens(0.0, 5) == 1.0
    assert A.expected_tokens(1.0, 5) == 6.0
    assert A.expected_tokens(0.5, 3) == pytest.approx(1 + 0.5 + 0.25 + 0.125, abs=1e-15)


def test_optimum_alpha_08_c_005():
    """alpha = 0.8, c = 0.05: the pages say N about 5-7 and 3.2x.  The formula
    peaks at N* = 8 with 3.092x; N = 5..7 give 2.951..3.082x, all within 5% of
    the peak (consistent within the curve's flatness; 3.2 is 3.5% above)."""
    n_star, s_star = A.best_n(0.8, 0.05)
    assert n_star == 8 and s_star == pytest.approx(3.0921, abs=1e-3)
    for n, s in [(5, 2.951), (6, 3.040), (7, 3.082)]:
        assert A.speedup(0.8, 0.05, n) == pytest.approx(s, abs=1e-3)
        assert A.speedup(0.8, 0.05, n) > 0.95 * s_star


def test_optimum_alpha_095_c_002_not_reproduced():
    """alpha = 0.95, c = 0.02: the pages say N about 8-10 and about 5x; the
    printed formula gives N* = 31 (9.95x) and 6.4-7.2x at N = 8-10.  The
    claim is recorded as not reproduced by the formula."""
    n_star, s_star = A.best_n(0.95, 0.02)
    assert n_star == 31 and s_star == pytest.approx(9.954, abs=1e-3)
    assert [round(A.speedup(0.95, 0.02, n), 3) for n in (8, 9, 10)] == [6.375, 6.801, 7.187]


def test_alpha_lever_at_n5():
    """N = 5, alpha 0.6 -> 0.9: the pages print 2.2 -> 4.1 tokens per call;
    the formula gives 2.383 -> 4.686 (recorded discrepancy).  Passo 6's
    'alpha about 0.9 gives 4-5 tokens per call' holds for N = 4..5."""
    assert A.expected_tokens(0.6, 5) == pytest.approx(2.383, abs=1e-3)
    assert A.expected_tokens(0.9, 5) == pytest.approx(4.686, abs=1e-3)
    assert 4.0 <= A.expected_tokens(0.9, 4) <= 5.0 and 4.0 <= A.expected_tokens(0.9, 5) <= 5.0


def test_exercise2_curve():
    """Exercicios 2: alpha = 0.9, c = 0.04, N = 1..10: tokens per call rise
    and the speed-up rises monotonically to 4.901 at N = 10 (the global
    optimum, N = 15, gives 5.092)."""
    s = [A.speedup(0.9, 0.04, n) for n in range(1, 11)]
    assert all(b > a for a, b in zip(s, s[1:]))
    assert s[-1] == pytest.approx(4.901, abs=1e-3)
    n_star, s_star = A.best_n(0.9, 0.04)
    assert n_star == 15 and s_star == pytest.approx(5.092, abs=1e-3)


@pytest.mark.parametrize("c", [0.01, 0.1, 0.3, 0.7])
def test_break_even_alpha_gt_c(c):
    """[ZH] section 2: speculation pays when alpha > c; exact for N = 1:
    speed-up (1 + alpha) / (1 + c) > 1 iff alpha > c."""
    for alpha in [c - 0.005, c + 0.005]:
        assert (A.speedup(alpha, c, 1) > 1.0) == (alpha > c)
