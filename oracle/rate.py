"""RateQuant bit allocation, plain Python (TEST INFRASTRUCTURE ONLY: tests and
the benchmark's CPU leg may use it; the library has its own implementation).

Follows the RateQuant technical summary (gist.science), methodology:
  * step 1: per-component distortion-rate model D_i(b) = alpha_i beta_i^-b,
    minimise sum_i w_i D_i(b_i) subject to sum_i b_i = B; the Lagrange
    stationarity condition gives the reverse water-filling solution;
  * step 3: integer bit widths by a greedy marginal-gain loop (the page's
    Algorithm 1), per-quantizer (alpha, beta) fitted from five bit widths
    ("distortion calibration"), keys and values as separate components
    ("K/V separation").
Readings where the page is silent are stated at each function.
"""
from __future__ import annotations

import math


def fit_rate_distortion(bits, mse):
    """(alpha, beta) of D(b) = alpha beta^-b from measured (b, mse) points.

    Reading: ordinary least squares on ln mse = ln alpha - b ln beta (the page
    fits the model at five bit widths and names no loss).
    """
    n = len(bits)
    if n < 2 or len(mse) != n or any(m <= 0 for m in mse):
        raise ValueError("need >= 2 points with positive mse")
    y = [math.log(m) for m in mse]
    mb = sum(bits) / n
    my = sum(y) / n
    sbb = sum((b - mb) ** 2 for b in bits)
    if sbb == 0:
        raise ValueError("bit widths must differ")
    slope = sum((b - mb) * (v - my) for b, v in zip(bits, y)) / sbb
    intercept = my - slope * mb
    return math.exp(intercept), math.exp(-slope)


def waterfill(alpha, beta, w, total_bits):
    """Real-valued optimum b_i of sum w_i alpha_i beta_i^-b_i with sum b_i = B.

    Stationarity: w_i alpha_i ln(beta_i) beta_i^-b_i = lambda for every i, so
    b_i = (ln(w_i alpha_i ln beta_i) - ln lambda) / ln beta_i, and the budget
    fixes ln lambda.  With one common (alpha, beta) this is the page's
    b_i = b_mean + (ln w_i - ln w_geo) / ln beta.  No clipping to a range.
    """
    n = len(w)
    lb = [math.log(bt) for bt in beta]
    c = [math.log(w[i] * alpha[i] * lb[i]) for i in range(n)]
    ln_lambda = (sum(c[i] / lb[i] for i in range(n)) - total_bits) / sum(1.0 / x for x in lb)
    return [(c[i] - ln_lambda) / lb[i] for i in range(n)]


def allocate_greedy(alpha, beta, w, allowed, total_bits):
    """Integer bit widths from the allowed set, sum <= B.

    Reading of the greedy marginal-gain loop: every component starts at the
    smallest allowed width; while budget remains, the component whose next
    allowed width buys the largest weighted distortion reduction per bit
    (and still fits the remaining budget) takes that step; ties go to the
    lowest index.  Steps of more than one bit are scored per bit.
    """
    levels = sorted(set(int(a) for a in allowed))
    n = len(w)
    b = [levels[0]] * n
    left = total_bits - n * levels[0]
    if left < 0:
        raise ValueError("budget below the smallest width")

    def dist(i, x):
        return w[i] * alpha[i] * beta[i] ** (-x)

    while True:
        best, best_gain = -1, 0.0
        for i in range(n):
            k = levels.index(b[i])
            if k + 1 >= len(levels):
                continue
            step = levels[k + 1] - b[i]
            if step > left:
                continue
            gain = (dist(i, b[i]) - dist(i, levels[k + 1])) / step
            if best < 0 or gain > best_gain:
                best, best_gain = i, gain
        if best < 0:
            return b
        k = levels.index(b[best])
        left -= levels[k + 1] - b[best]
        b[best] = levels[k + 1]
