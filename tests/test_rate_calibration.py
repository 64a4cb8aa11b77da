"""RateQuant distortion calibration on this cache's own quantizers (RateQuant
technical summary, methodology step 3 "distortion calibration" and "K/V
separation", pipeline step 2), then allocation per (layer, KV head) and a
cache table built from it.

CPU tests.  The MSE of each quantizer is measured on synthetic keys and values
shaped like the Llama-3-8B workload (per-channel asymmetric keys in groups of
32 tokens, per-token asymmetric values in groups of 32 channels) at the
widths the cache implements, 2, 3, 4 and 8 bits (the page fits five widths;
the library has four).  The codes are the oracle's, which the GPU parity
tests hold bit-identical to the library's; tests/test_gpu_parity.py also
measures the same MSE from the library's packed records.
"""
import math

import numpy as np
import pytest

import oracle as O
from decode_attention_quantize_amd import build as kb
from decode_attention_quantize_amd import kvq as K
from oracle import rate as R
from synth import workloads as W

WIDTHS = (2, 3, 4, 8)


@pytest.fixture(scope="module", autouse=True)
def built():
    if kb.is_stale():
        kb.build()
    K.lib()


def calibration_mse(wl, layer, units, T, bits):
    """Mean squared error of the dequantized body keys and values (outside the
    fp16 window) over the given units, with both tensors at `bits`."""
    sc = O.scheme_for(wl.with_(fixed_pairs=((bits, bits),) * wl.L), layer)
    s_eff, nb, _ = O.state_prefill(T, wl.sinks, wl.window, wl.flush)
    ek = ev = 0.0
    for u in units:
        b, h = divmod(u, wl.Hkv)
        Kx, Vx = O.unit_inputs(wl, layer, b, h, T)
        enc = O.encode_unit(sc, Kx, Vx, T, s_eff, nb)
        Kh, Vh = O.dequant_unit(sc, Kx, enc, T, s_eff, nb)
        kt = O.f16_to_f64(Kx[s_eff:s_eff + nb])
        vt = O.f16_to_f64(Vx[s_eff:s_eff + nb])
        ek += float(np.mean((Kh[s_eff:s_eff + nb] - kt) ** 2))
        ev += float(np.mean((Vh[s_eff:s_eff + nb] - vt) ** 2))
    return ek / len(units), ev / len(units)


@pytest.fixture(scope="module")
def calibration():
    wl = W.C3
    units = [0, 9, 37]
    mse = {b: calibration_mse(wl, 0, units, 512, b) for b in WIDTHS}
    return wl, mse


def test_distortion_follows_the_grid_step(calibration):
    """Asymmetric uniform quantization on a group's min..max range: the step
    is range / (2^b - 1), and the MSE, about step^2 / 12 (the two group
    extremes are exact at every width), falls between widths b0 < b1 by
    ((2^b1 - 1) / (2^b0 - 1))^2: 5.44 from 2 to 3 bits, 4.59 from 3 to 4,
    289 from 4 to 8."""
    _, mse = calibration
    for t in (0, 1):
        m = [mse[b][t] for b in WIDTHS]
        assert all(m[i] > m[i + 1] for i in range(len(m) - 1)), m
        for b0, b1, tol in ((2, 3, 0.12), (3, 4, 0.12), (4, 8, 0.3)):
            predicted = ((2 ** b1 - 1) / (2 ** b0 - 1)) ** 2
            ratio = mse[b0][t] / mse[b1][t]
            assert abs(ratio / predicted - 1) < tol, (t, b0, b1, ratio, predicted)


def test_fit_on_the_quantizers_matches_the_allocation_oracle(calibration):
    _, mse = calibration
    for t in (0, 1):
        pts = [mse[b][t] for b in WIDTHS]
        a, beta = K.kvq_fit_rate_distortion(list(WIDTHS), pts)
        ao, bo = R.fit_rate_distortion(list(WIDTHS), pts)
        assert math.isclose(a, ao, rel_tol=1e-12) and math.isclose(beta, bo, rel_tol=1e-12)
        assert 3.0 < beta < 5.5
        # the fitted model reproduces every measured point within the scatter
        # of a least-squares line through four points
        for b in WIDTHS:
            assert 0.5 < a * beta ** (-b) / mse[b][t] < 2.0, (t, b)


def sensitivities(L, H, seed=7):
    """Seeded per-(layer, KV head, K/V) sensitivities: higher in the first and
    last layers (the U-shape the page reports for gradient sensitivities),
    keys above values, log-normal spread across heads.  Real values need model
    gradients, which this build has no access to."""
    r = np.random.default_rng(seed)
    x = np.linspace(-1.0, 1.0, L)
    layer = 1.0 + 2.0 * x ** 2
    w = np.empty((L, H, 2))
    w[..., 0] = 2.0 * layer[:, None] * np.exp(0.5 * r.normal(size=(L, H)))
    w[..., 1] = 1.0 * layer[:, None] * np.exp(0.5 * r.normal(size=(L, H)))
    return w


def test_per_head_allocation_builds_a_cache_table(calibration):
    """Components = keys and values of every (layer, KV head); the library's
    greedy allocation equals the oracle's; the per-head table becomes a cache
    whose layers are (layer, KV head) pairs of one KV head each, and the
    cache's f_m equals the mean allocated width."""
    wl, mse = calibration
    L, H = wl.L, wl.Hkv
    fits = [K.kvq_fit_rate_distortion(list(WIDTHS), [mse[b][t] for b in WIDTHS]) for t in (0, 1)]
    w = sensitivities(L, H)
    alpha = [fits[t][0] for l in range(L) for h in range(H) for t in (0, 1)]
    beta = [fits[t][1] for l in range(L) for h in range(H) for t in (0, 1)]
    ww = w.reshape(-1).tolist()
    budget = 4 * 2 * L * H                         # 4 bits per tensor on average
    allowed = (2, 4, 8)
    bits = K.kvq_allocate_bits(alpha, beta, ww, allowed, budget)
    assert bits == R.allocate_greedy(alpha, beta, ww, allowed, budget)
    assert sum(bits) <= budget and set(bits) <= set(allowed)
    b = np.array(bits).reshape(L, H, 2)
    # more sensitive components never get fewer bits than less sensitive ones
    # of the same kind (same distortion model)
    for t in (0, 1):
        order = np.argsort(w[..., t].ravel())
        assert np.all(np.diff(b[..., t].ravel()[order]) >= 0)
    pairs = [(int(b[l, h, 0]), int(b[l, h, 1])) for l in range(L) for h in range(H)]
    cfg = K.make_config(wl.B, wl.gq, 1, L * H, wl.T + wl.steps)
    handle = K.kvq_create(cfg, pairs)
    try:
        f_m, _ = K.kvq_average_bits(handle)
        assert f_m == sum(bits) / len(bits)
    finally:
        K.kvq_destroy(handle)
