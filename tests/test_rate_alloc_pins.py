"""Pins of the RateQuant allocation oracle (oracle/rate.py) against closed
forms, invariants and brute force (RateQuant technical summary, methodology
steps 1 and 3)."""
import itertools
import math

import numpy as np
import pytest

from oracle import rate as R


def test_fit_recovers_exact_model_and_least_squares():
    bits = [2, 3, 4, 6, 8]
    for alpha, beta in ((0.7, 3.6), (2.5, 5.3), (1e-3, 4.0)):
        a, b = R.fit_rate_distortion(bits, [alpha * beta ** (-x) for x in bits])
        assert math.isclose(a, alpha, rel_tol=1e-12) and math.isclose(b, beta, rel_tol=1e-12)
    # noisy data: the residuals of the log-linear fit are orthogonal to [1, b]
    r = np.random.default_rng(5)
    mse = [2.0 * 4.2 ** (-x) * math.exp(r.normal() * 0.2) for x in bits]
    a, b = R.fit_rate_distortion(bits, mse)
    res = [math.log(m) - (math.log(a) - x * math.log(b)) for x, m in zip(bits, mse)]
    assert abs(sum(res)) < 1e-12 and abs(sum(x * e for x, e in zip(bits, res))) < 1e-11


def test_waterfill_budget_and_stationarity():
    r = np.random.default_rng(6)
    n = 24
    alpha = list(r.uniform(0.2, 3.0, n))
    beta = list(r.uniform(3.0, 6.0, n))
    w = list(np.exp(r.normal(size=n)))
    B = 4.0 * n
    b = R.waterfill(alpha, beta, w, B)
    assert math.isclose(sum(b), B, rel_tol=1e-12)
    marg = [w[i] * alpha[i] * math.log(beta[i]) * beta[i] ** (-b[i]) for i in range(n)]
    assert max(marg) / min(marg) - 1 < 1e-10


def test_waterfill_common_model_is_the_printed_solution_and_am_gm_bound():
    # one (alpha, beta) for all: b_i = b_mean + (ln w_i - ln w_geo) / ln beta,
    # and the distortion ratio uniform/optimal equals AM(w)/GM(w)
    r = np.random.default_rng(7)
    w = list(np.exp(r.normal(size=10)))
    beta, alpha, bm = 4.7, 1.3, 3.5
    b = R.waterfill([alpha] * 10, [beta] * 10, w, bm * 10)
    lgeo = sum(math.log(x) for x in w) / 10
    for i in range(10):
        assert math.isclose(b[i], bm + (math.log(w[i]) - lgeo) / math.log(beta), rel_tol=1e-12)
    d_uni = sum(x * alpha * beta ** (-bm) for x in w)
    d_opt = sum(w[i] * alpha * beta ** (-b[i]) for i in range(10))
    am, gm = sum(w) / 10, math.exp(lgeo)
    assert math.isclose(d_uni / d_opt, am / gm, rel_tol=1e-12)


def _objective(alpha, beta, w, b):
    return sum(w[i] * alpha[i] * beta[i] ** (-b[i]) for i in range(len(w)))


def test_greedy_unit_steps_is_optimal_bruteforce():
    r = np.random.default_rng(8)
    levels = list(range(2, 9))
    for trial in range(40):
        n = 3
        alpha = list(r.uniform(0.2, 3.0, n))
        beta = list(r.uniform(3.0, 6.0, n))
        w = list(np.exp(r.normal(size=n) * 1.5))
        B = int(r.integers(3 * 2, 3 * 8 + 1))
        g = R.allocate_greedy(alpha, beta, w, levels, B)
        assert sum(g) == B
        best = min(_objective(alpha, beta, w, c) for c in itertools.product(levels, repeat=n) if sum(c) == B)
        assert math.isclose(_objective(alpha, beta, w, g), best, rel_tol=1e-12), (trial, g)


def test_greedy_matches_closed_form_when_it_is_integral():
    # w_i = beta^k_i with sum k_i = 0: the real solution is b_mean + k_i
    beta = 4.0
    ks = [-2, -1, 0, 0, 1, 2, 3, -3]
    w = [beta ** k for k in ks]
    n = len(w)
    b = R.waterfill([1.0] * n, [beta] * n, w, 5 * n)
    assert all(math.isclose(b[i], 5 + ks[i], abs_tol=1e-12) for i in range(n))
    g = R.allocate_greedy([1.0] * n, [beta] * n, w, range(2, 9), 5 * n)
    assert g == [5 + k for k in ks]


def test_greedy_respects_allowed_widths_and_budget():
    alpha, beta, w = [1.0] * 4, [4.0] * 4, [8.0, 1.0, 1.0, 0.1]
    g = R.allocate_greedy(alpha, beta, w, (2, 4, 8), 18)
    assert all(x in (2, 4, 8) for x in g) and sum(g) <= 18
    assert g[0] >= g[1] >= g[3]              # more sensitive, more bits
    with pytest.raises(ValueError):
        R.allocate_greedy(alpha, beta, w, (2, 4, 8), 7)
