"""Pins of the oracle's mixed 4/8-bit inner key groups (InnerQ, limitations and
future work: a hybrid of 4-bit and 8-bit groups).

Reading checked here: per token, the k_hi_groups inner groups whose 4-bit
quantizer has the largest step are quantized at 8 bits instead.  The pins use
routes other than the unit encoder: the per-group quantizers (pinned by brute
force elsewhere), a brute-force minimax over every choice of groups, hand-made
ties, the two uniform special cases, and the error reduction it must give.
"""
import itertools

import numpy as np
import pytest

import oracle as O
from synth import workloads as W

rng = np.random.default_rng(4242)


def h16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def _keys(n, loud=(5, 70), factor=12.0):
    """fp16 [n][128] keys: N(0,1) with a few loud channels and per-token
    scale changes, so that group steps differ within and across tokens."""
    k = rng.standard_normal((n, 128))
    for c in loud:
        k[:, c] *= factor
    k *= np.exp(rng.uniform(-2, 2, (n, 1)))
    return h16(k).reshape(n, 128)


def _encode(K, kg, m, bits=4, hybrid=1):
    n = K.shape[0]
    V = h16(rng.standard_normal((n, 128))).reshape(n, 128)
    sc = O.make_scheme(k_mode=1, k_group=kg, k_bits=bits, v_bits=4, k_hybrid=hybrid,
                       k_hi_groups=m)
    return sc, V, O.encode_unit(sc, K, V, n, 0, n)


def _group_quant(x16, bits, hybrid=1):
    if hybrid and O.hybrid_is_sym(x16, 1, 10):
        return O.quant_sym(x16, bits)
    return O.quant_asym(x16, bits)


@pytest.mark.parametrize("kg", [32, 64])
def test_mixed_reduces_to_uniform_widths(kg):
    K = _keys(48)
    ng = 128 // kg
    _, _, e4 = _encode(K, kg, 0)
    _, _, e8 = _encode(K, kg, 0, bits=8)
    _, _, m0 = _encode(K, kg, 0)
    _, _, mall = _encode(K, kg, ng)
    assert np.array_equal(m0["kcodes"], e4["kcodes"]) and np.array_equal(m0["kmeta"], e4["kmeta"])
    assert np.all(m0["kwidth"] == 4)
    assert np.array_equal(mall["kcodes"], e8["kcodes"]) and np.array_equal(mall["kmeta"], e8["kmeta"])
    assert np.all(mall["kwidth"] == 8)


@pytest.mark.parametrize("kg,m", [(32, 1), (32, 2), (32, 3), (64, 1)])
def test_mixed_choice_is_minimax_over_all_choices(kg, m):
    # for every token: the largest quantization step over its groups, after
    # the chosen groups move to 8 bits, is the smallest any choice of m groups
    # reaches (brute force over all of them), and each group's codes and
    # parameters are those of the per-group quantizer at its width
    K = _keys(40)
    ng = 128 // kg
    _, _, enc = _encode(K, kg, m)
    for t in range(K.shape[0]):
        st = {}
        ref = {}
        for g in range(ng):
            for b in (4, 8):
                codes, meta = _group_quant(K[t, g * kg:(g + 1) * kg], b)
                st[g, b] = int(meta[0]) & 0x7FFF
                ref[g, b] = (codes, meta)
        hi = [g for g in range(ng) if enc["kwidth"][t, g] == 8]
        assert len(hi) == m and all(enc["kwidth"][t, g] in (4, 8) for g in range(ng))
        cost = lambda S: max(st[g, 8 if g in S else 4] for g in range(ng))
        best = min(cost(set(S)) for S in itertools.combinations(range(ng), m))
        assert cost(set(hi)) == best, (t, hi)
        # no group left at 4 bits has a larger 4-bit step than a chosen one
        assert min(st[g, 4] for g in hi) >= max([st[g, 4] for g in range(ng) if g not in hi] or [0])
        for g in range(ng):
            codes, meta = ref[g, int(enc["kwidth"][t, g])]
            assert np.array_equal(enc["kcodes"][t, g * kg:(g + 1) * kg], codes), (t, g)
            assert np.array_equal(enc["kmeta"][t, g], meta), (t, g)


def test_mixed_equal_steps_choose_the_lower_group():
    row = rng.standard_normal(64)
    k = np.concatenate([row, row])                       # groups 0 and 1 identical
    louder = np.concatenate([row, 3.0 * row])            # group 1 has the larger step
    K = h16(np.stack([k, louder])).reshape(2, 128)
    _, _, enc = _encode(K, 64, 1)
    assert enc["kwidth"].tolist() == [[8, 4], [4, 8]]
    # four groups of 32, steps tied in pairs: groups (1, 3) share the largest
    r32 = rng.standard_normal(32)
    K4 = h16(np.concatenate([r32, 4 * r32, r32, 4 * r32])[None]).reshape(1, 128)
    _, _, e1 = _encode(K4, 32, 1)
    _, _, e3 = _encode(K4, 32, 3)
    assert e1["kwidth"].tolist() == [[4, 8, 4, 4]]
    assert e3["kwidth"].tolist() == [[8, 8, 4, 8]]


def test_mixed_dequant_uses_each_groups_width():
    K = _keys(32)
    sc, V, enc = _encode(K, 64, 1)
    Kh, _ = O.dequant_unit(sc, K, enc, 32, 0, 32)
    for t in (0, 7, 31):
        for g in range(2):
            b = int(enc["kwidth"][t, g])
            s, z = enc["kmeta"][t, g]
            want = [O.dequant(int(c), int(s), int(z), b) for c in enc["kcodes"][t, 64 * g:64 * g + 64]]
            assert np.array_equal(Kh[t, 64 * g:64 * g + 64], want)


def test_mixed_error_sits_between_uniform_4_and_8_bits():
    # the 8-bit groups shrink the error of the groups that dominated it
    wl = W.C5.with_(B=1, Hq=8, T=256, steps=1, k_out_count=2, v_out_count=0)
    K, V = O.unit_inputs(wl, 0, 0, 0, 256)
    k = K.view(np.float16).astype(np.float64)
    errs = {}
    for name, bits, m in (("k4", 4, 0), ("mixed", 4, 1), ("k8", 8, 0)):
        sc = O.make_scheme(k_mode=1, k_group=64, k_bits=bits, v_bits=2, k_hybrid=1, k_hi_groups=m)
        enc = O.encode_unit(sc, K, V, 256, 0, 256)
        Kh, _ = O.dequant_unit(sc, K, enc, 256, 0, 256)
        errs[name] = np.mean((Kh - k) ** 2)
    assert errs["k8"] < errs["mixed"] < 0.5 * errs["k4"], errs


def test_mixed_rejects_what_it_does_not_define():
    K = _keys(8)
    V = h16(rng.standard_normal((8, 128))).reshape(8, 128)
    for kw in (dict(k_mode=0, k_group=32, k_hi_groups=1),           # per-channel keys
               dict(k_mode=1, k_group=64, k_bits=2, k_hi_groups=1),  # not 4-bit keys
               dict(k_mode=1, k_group=64, k_hi_groups=3),            # more groups than a token has
               dict(k_mode=1, k_group=64, k_hi_groups=1, outliers=2)):
        sc = O.make_scheme(**{"v_bits": 4, **kw})
        with pytest.raises(ValueError):
            O.encode_unit(sc, K, V, 8, 0, 0 if kw["k_mode"] == 0 else 8)
