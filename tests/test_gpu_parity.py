"""GPU path vs the CPU oracle: codes, parameters, outliers and fp16 windows
bit-exact; attention outputs within 2e-3 (row-max-normalised) at every decode
step, always through the compressed cache (prefill, then token by token)."""
import numpy as np
import pytest
import torch

from gpu_harness import TOL, check_unit, check_units, run_gpu, say
from synth import workloads as W

pytestmark = pytest.mark.gpu

REDUCED = {
    "C1": W.C1,
    "C2r": W.C2.with_(Hq=4, Hkv=4, T=1024),                       # flushes at steps 4 and 36
    "C2r-peaky": W.C2.with_(Hq=2, Hkv=2, T=1024, steps=8, q_scale=4.0),
    "C3r": W.C3.with_(L=5, B=2, Hq=8, Hkv=2, T=512, steps=40, fixed_pairs=W.PAIR_SET),
    "C4r": W.C4.with_(Hq=2, Hkv=2, T=1024, steps=33),             # one flush at step 32
    "C5r": W.C5.with_(B=2, Hq=16, Hkv=2, T=500, steps=4),          # ragged last block
    "C5r-whole-blocks": W.C5.with_(B=2, Hq=16, Hkv=2, T=512, steps=3),
    # InnerQ key normalization on C5's inner groups; one key channel x64
    "C5rn": W.C5.with_(B=2, Hq=16, Hkv=2, T=500, steps=4, k_norm=True, k_out_factor=64.0),
    # the Hadamard 2-bit page's pairing: KIVI int4 keys (per channel) with
    # rotated 2-bit values, and its ternary-value negative control
    "P5r": W.C2.with_(Hq=4, Hkv=4, T=1024, steps=8, v_hadamard=True, v_out_count=2),
    "P5r-ternary": W.C2.with_(Hq=4, Hkv=4, T=1024, steps=8, v_ternary=True, v_out_count=2),
    # InnerQ's mixed 4/8-bit groups: one of each token's two key groups at 8
    # bits (matrix-core kernel), and two of four groups of 32 (LDS-staged)
    "C5rm": W.C5.with_(B=2, Hq=16, Hkv=2, T=500, steps=4, k_hi_groups=1, k_out_count=2),
    "C5rm32": W.C5.with_(B=2, Hq=16, Hkv=2, T=300, steps=3, k_group=32, k_hi_groups=2),
}

EDGE = {
    "short-prompt-all-sinks": W.C2.with_(Hq=2, Hkv=2, T=3, steps=5),
    # a prompt shorter than the sinks: the first appends complete the sinks,
    # later ones fill the window until it flushes a block (step 65)
    "short-prompt-sinks-then-flush": W.C2.with_(Hq=2, Hkv=2, T=3, window=32, steps=70),
    # the same with inner key groups (no window: tokens past the sinks are
    # quantized at once)
    "inner-short-prompt-sinks": W.C5.with_(B=1, Hq=8, Hkv=1, T=2, sinks=4, steps=6),
    "window-only": W.C1.with_(T=40),
    "one-block": W.C1.with_(T=64),
    "inner-single-token": W.C5.with_(B=1, Hq=8, Hkv=1, T=1, steps=3),
    "uniform-3bit": W.C2.with_(Hq=2, Hkv=2, T=300, steps=3, fixed_pairs=((3, 3),)),
    "gqa2-kv8": W.C3.with_(L=1, B=1, Hq=4, Hkv=2, T=200, steps=2, fixed_pairs=((8, 8),)),
    "gqa16": W.C3.with_(L=1, B=1, Hq=16, Hkv=1, T=300, steps=2, fixed_pairs=((4, 2),)),
    "knorm-window-only": W.C5.with_(B=1, Hq=8, Hkv=1, T=20, steps=3, k_norm=True),
    "knorm-sinks-window": W.C5.with_(B=1, Hq=8, Hkv=1, T=300, steps=3, sinks=4, window=32,
                                     k_norm=True, k_out_factor=64.0),
    "mixed-single-token": W.C5.with_(B=1, Hq=8, Hkv=1, T=1, steps=3, k_hi_groups=1),
    "mixed-all-8bit": W.C5.with_(B=1, Hq=8, Hkv=1, T=100, steps=2, k_hi_groups=2),
    "mixed-mha-v4": W.C5.with_(B=1, Hq=4, Hkv=4, T=200, steps=2, k_hi_groups=1, v_hadamard=False,
                               fixed_pairs=((4, 4),)),
    "mixed-gqa4-knorm-window": W.C5.with_(B=1, Hq=8, Hkv=2, T=300, steps=3, sinks=4, window=32,
                                          k_norm=True, k_hi_groups=1, k_out_factor=64.0),
    # eight groups of 16 per token, three of them at 8 bits (LDS-staged kernel)
    "mixed-g16": W.C5.with_(B=1, Hq=8, Hkv=1, T=100, steps=2, k_group=16, k_hi_groups=3),
    # a 2-bit-key layer ignores the setting (plain inner 2-bit keys)
    "mixed-ignored-k2": W.C5.with_(B=1, Hq=8, Hkv=1, T=100, steps=2, k_hi_groups=1, fixed_pairs=((2, 2),)),
    # eight query rows over 8-bit values with loud value channels (x4000): large value
    # scales against the weights' lift for 8-bit groups
    "gqa8-kv8-loud-values": W.C3.with_(L=1, B=1, Hq=8, Hkv=1, T=300, steps=2, fixed_pairs=((8, 8),),
                                       v_out_count=4, v_out_factor=4000.0),
    # peaked attention (queries x3) over 4-bit values: most weights far below the row
    # ceiling, the subnormal range the lift for 4-bit groups guards against
    "gqa4-k4v4-peaky": W.C3.with_(L=1, B=1, Hq=4, Hkv=1, T=600, steps=2, fixed_pairs=((4, 4),),
                                  q_scale=3.0),
    # the same over 8-bit values with eight rows, and over MHA 8-bit values
    "gqa8-kv8-peaky": W.C3.with_(L=1, B=1, Hq=8, Hkv=1, T=600, steps=2, fixed_pairs=((8, 8),),
                                 q_scale=3.0),
    "mha-kv8-peaky": W.C2.with_(Hq=2, Hkv=2, T=600, steps=2, fixed_pairs=((8, 8),), q_scale=3.0),
    # single-row layers with the key and value products packed into rows 0 and 1 of the
    # matrix-core tiles, at the other key/value widths (2-bit keys with 8-bit values and
    # the reverse), with sinks, a window and a flush during the decode steps
    "mha-k2v8": W.C2.with_(Hq=2, Hkv=2, T=700, steps=40, fixed_pairs=((2, 8),)),
    "mha-k8v2": W.C2.with_(Hq=2, Hkv=2, T=700, steps=40, fixed_pairs=((8, 2),)),
}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_all(name, wl):
    say(f"[parity] {name}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} L={wl.L} T={wl.T} steps={wl.steps}")
    cache, outs = run_gpu(wl)
    worst = 0.0
    for l in range(wl.L):
        for u in range(wl.units):
            worst = max(worst, check_unit(wl, cache, outs, l, u, label=f"{name} l{l} u{u}"))
    say(f"[parity] {name}: worst row error {worst:.3e}")
    cache.close()


@pytest.mark.parametrize("name", list(REDUCED))
def test_reduced_configs(name):
    _check_all(name, REDUCED[name])


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases(name):
    _check_all(name, EDGE[name])


@pytest.mark.parametrize("name", ["C1", "C2r", "C3r", "C4r", "C5r", "C5rn", "P5r", "P5r-ternary", "C5rm"])
def test_reduced_configs_general_kernel(name, monkeypatch):
    """The same workloads through the LDS-staged decode kernel (the path every
    scheme the matrix-core kernel does not cover takes)."""
    monkeypatch.setenv("KVQ_DECODE_KERNEL", "generic")
    _check_all(name + "/general", REDUCED[name])


def test_generator_matches_cpu():
    wl = W.C4
    a = wl.k(0, 0, 1, 3, 5, 1000, 1100, device="cuda").cpu()
    b = wl.k(0, 0, 1, 3, 5, 1000, 1100)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    a = W.C5.v(0, 1, 2, 0, 8, 0, 40, device="cuda").cpu()
    b = W.C5.v(0, 1, 2, 0, 8, 0, 40)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_capacity_and_state_errors_on_device_cache():
    from decode_attention_quantize_amd import KVQCache, KVQError, config_from_workload
    wl = W.C1.with_(T=64)
    cache = KVQCache(config_from_workload(wl, max_tokens=64), wl.bit_pairs(), device="cuda")
    q = wl.q(0, 0, device="cuda")
    with pytest.raises(KVQError):
        cache.decode(0, q)                                   # before prefill
    k = wl.k(0, 0, 1, 0, 1, 0, 64, device="cuda").contiguous()
    v = wl.v(0, 0, 1, 0, 1, 0, 64, device="cuda").contiguous()
    cache.prefill(0, k, v)
    with pytest.raises(KVQError) as e:
        cache.append(0, k[:, :, 0].contiguous(), v[:, :, 0].contiguous())
    assert e.value.status == 2                               # capacity
    assert cache.state(0) == (64, 0, 32, 32)
    out = cache.decode(0, q)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    cache.prefill(0, k[:, :, :0].contiguous(), v[:, :, :0].contiguous())   # T = 0
    with pytest.raises(KVQError) as e:
        cache.decode(0, q)
    assert e.value.status == 4
    cache.close()


# ---------------------------------------------------------------- stale buffers, status paths
@pytest.mark.parametrize("name", ["C5r", "C5rm", "C5rm32", "C2r", "C4r", "C3r"])
def test_stale_buffer_contents_never_reach_the_output(name):
    """Layer buffers filled with 0xFF (fp16 NaN patterns) before the prefill:
    outputs still match the oracle, and the per-token sections of the slots
    past the last token of a partly filled block hold zeros."""
    wl = REDUCED[name]
    say(f"[stale] {name}: buffers pre-filled with 0xff")
    cache, outs = run_gpu(wl, fill=0xFF)
    worst = 0.0
    for l in range(wl.L):
        for u in range(wl.units):
            worst = max(worst, check_unit(wl, cache, outs, l, u, label=f"{name}/0xff l{l} u{u}",
                                          check_tail=True))
    say(f"[stale] {name}: worst row error {worst:.3e}")
    assert cache.nonfinite_rows() == 0
    cache.close()


def test_nonfinite_rows_are_counted():
    """|q_c s_c| beyond binary16 with per-channel keys is outside the decode's
    domain: the affected rows are counted in the workspace, and the count
    resets when read."""
    from decode_attention_quantize_amd import KVQCache, config_from_workload
    wl = W.C1.with_(k_out_factor=300.0)
    cache = KVQCache(config_from_workload(wl), wl.bit_pairs(), device="cuda")
    k = wl.k(0, 0, 1, 0, 1, 0, wl.T, device="cuda").contiguous()
    v = wl.v(0, 0, 1, 0, 1, 0, wl.T, device="cuda").contiguous()
    cache.prefill(0, k, v)
    q = wl.q(0, 0, device="cuda").contiguous()
    cache.decode(0, q)
    assert cache.nonfinite_rows() == 0
    out = cache.decode(0, (q.float() * 4000.0).half())   # q_c s_c ~ 1e6 on the loud channels
    n = cache.nonfinite_rows()
    assert n == 1 and not torch.isfinite(out).all(), n
    assert cache.nonfinite_rows() == 0
    cache.close()


def _ties_tensor(T, D, bits, step, token_groups, nudge, glen=32):
    """fp16 [T][D] whose groups (32 tokens of a channel when token_groups, else
    glen channels of a token) hold their minimum and maximum at positions 0
    and 1 and elsewhere base + step * m, m a multiple of 1/2 in [0, Q]: with
    s = step exactly, every quotient (x - min) / s is m, so half the elements
    sit on a rounding tie; `nudge` moves every fifth of those one ulp up, to a
    hair above the tie."""
    Q = (1 << bits) - 1
    t = np.arange(T)[:, None]
    c = np.arange(D)[None, :]
    pos = (t % 32) if token_groups else (c % glen)
    m = ((t * 7 + c * 3) % (2 * Q + 1)) * 0.5
    m = np.where(pos == 0, 0.0, np.where(pos == 1, float(Q), m))
    base = -1.0 + 0.25 * ((c % 4) if token_groups else (t % 4))
    x = (base + step * m).astype(np.float16)
    if nudge:
        hit = (pos >= 2) & ((t + c) % 5 == 0) & (m != np.floor(m))
        x = np.where(hit, np.nextafter(x, np.float16(np.inf)), x)
    return x


@pytest.mark.parametrize("keys", ["channel", "channel-rotated", "inner"])
@pytest.mark.parametrize("pair", [(2, 2), (4, 4), (8, 2), (2, 8)])
@pytest.mark.parametrize("nudge", [False, True])
def test_prefill_codes_on_rounding_ties(keys, pair, nudge):
    """Quotients exactly on (or one ulp past) a half-integer, where a
    reciprocal estimate cannot decide the rounding: the library's codes and
    parameters equal the oracle's correctly rounded ones bit for bit (keys
    per channel, also beside Hadamard-rotated values -- the rotation moves
    the values off their ties, the keys keep them -- or in inner groups of
    64 with the symmetric/asymmetric choice)."""
    import oracle as O
    from decode_attention_quantize_amd import KVQCache, config_from_workload
    from gpu_harness import HostLayer, unit_body
    from kvq_unpack import unpack_unit
    kb, vb = pair
    if keys == "channel":
        wl = W.C1.with_(name="ties", window=0, fixed_pairs=(pair,), T=256)
    elif keys == "channel-rotated":
        wl = W.C1.with_(name="ties-rotated", window=0, fixed_pairs=(pair,), T=256, v_hadamard=True)
    else:
        wl = W.C5.with_(name="ties-inner", B=1, Hq=1, Hkv=1, T=256, steps=1, v_hadamard=False,
                        fixed_pairs=(pair,))
    T, D = wl.T, wl.D
    K = _ties_tensor(T, D, kb, 2.0 ** -6 if kb == 8 else 0.125, keys != "inner", nudge,
                     glen=wl.k_group if keys == "inner" else 32)
    V = _ties_tensor(T, D, vb, 2.0 ** -6 if vb == 8 else 0.125, False, nudge)
    say(f"[ties] {keys} keys, pair {pair} nudge {nudge}")
    cache = KVQCache(config_from_workload(wl), wl.bit_pairs(), device="cuda")
    k = torch.from_numpy(K).view(1, 1, T, D).cuda()
    v = torch.from_numpy(V).view(1, 1, T, D).cuda()
    cache.prefill(0, k, v)
    torch.cuda.synchronize()
    s_eff, nb, _ = O.state_prefill(T, wl.sinks, wl.window, wl.flush)
    enc = O.encode_unit(O.scheme_for(wl, 0), K.view(np.uint16), V.view(np.uint16), T, s_eff, nb)
    body, lay = unit_body(cache, 0, 0, HostLayer(cache, 0))
    got = unpack_unit(body, lay, kb, vb, nb, keys == "inner", wl.k_group, wl.v_group, wl.outliers, 0)
    for key in ("kcodes", "kmeta", "vcodes", "vmeta"):
        bad = np.argwhere(got[key] != enc[key])
        assert bad.size == 0, (pair, nudge, key, bad[:5].tolist())
    # the construction does reach the ties it is meant to
    assert np.any(enc["kcodes"] % 2 == 0) and np.any(enc["vcodes"] % 2 == 0)
    cache.close()


def _ternary_tie_values(T, D):
    """fp16 [T][D] whose per-token groups of 32 channels put elements on the
    ternary threshold |x| = s / 2 (s = the group's max |x|), one ulp either
    side of it, at +-s and at 0, over scales from 2^-20 (subnormal halves)
    to 2^4."""
    rng = np.random.default_rng(11)
    out = np.zeros((T, D), np.float32)
    for t in range(T):
        for g in range(D // 32):
            sc = np.float16(2.0 ** rng.integers(-20, 5) * (1 + rng.integers(0, 1024) / 1024))
            half = np.float16(sc / np.float16(2))
            cand = [sc, half, np.nextafter(half, np.float16(np.inf)), np.nextafter(half, np.float16(0)), np.float16(0)]
            x = np.array([cand[i] for i in rng.integers(0, len(cand), 32)], np.float16)
            x[rng.integers(0, 32)] = sc
            x *= np.where(rng.integers(0, 2, 32) == 1, np.float16(-1), np.float16(1)).astype(np.float16)
            out[t, 32 * g:32 * g + 32] = x.astype(np.float32)
    return out.astype(np.float16)


def test_prefill_ternary_values_on_their_threshold():
    """Ternary value groups (levels -s, 0, s) whose elements sit exactly on
    the rounding threshold |x| = s / 2 (which rounds to 0), one ulp past or
    short of it: the library's codes and (s, z) equal the oracle's bit for
    bit."""
    import oracle as O
    from decode_attention_quantize_amd import KVQCache, config_from_workload
    from gpu_harness import HostLayer, unit_body
    from kvq_unpack import unpack_unit
    wl = W.C1.with_(name="ternary-threshold", window=0, fixed_pairs=((4, 2),), T=256, v_ternary=True)
    T, D = wl.T, wl.D
    K = (np.random.default_rng(3).standard_normal((T, D))).astype(np.float16)
    V = _ternary_tie_values(T, D)
    say("[ternary threshold] C1 layout, K4 V2 ternary")
    cache = KVQCache(config_from_workload(wl), wl.bit_pairs(), device="cuda")
    k = torch.from_numpy(K).view(1, 1, T, D).cuda()
    v = torch.from_numpy(V).view(1, 1, T, D).cuda()
    cache.prefill(0, k, v)
    torch.cuda.synchronize()
    s_eff, nb, _ = O.state_prefill(T, wl.sinks, wl.window, wl.flush)
    enc = O.encode_unit(O.scheme_for(wl, 0), K.view(np.uint16), V.view(np.uint16), T, s_eff, nb)
    body, lay = unit_body(cache, 0, 0, HostLayer(cache, 0))
    got = unpack_unit(body, lay, 4, 2, nb, False, wl.k_group, wl.v_group, wl.outliers, 0)
    for key in ("kcodes", "kmeta", "vcodes", "vmeta"):
        bad = np.argwhere(got[key] != enc[key])
        assert bad.size == 0, (key, bad[:5].tolist())
    # all three levels occur
    assert all(np.any(enc["vcodes"] == c) for c in (0, 1, 2))
    cache.close()


def _hybrid_boundary_keys(T, D):
    """fp16 [T][D] whose inner key groups of 64 channels sit on the hybrid
    test's boundary for the ratio 1/10: minimum -1, maximum 4, 29 ones and
    zeros elsewhere give 10 |sum| = 320 = 64 (max - min) exactly (symmetric);
    one of the ones moved an ulp up (asymmetric) or down (symmetric).  Each
    group is scaled by a power of two, negated in turn, and its channels are
    permuted."""
    rng = np.random.default_rng(7)
    out = np.zeros((T, D), np.float32)
    for t in range(T):
        for g in range(D // 64):
            x = np.zeros(64, np.float32)
            x[0], x[1], x[2:31] = -1.0, 4.0, 1.0
            kind = (2 * t + g) % 3
            if kind == 1:
                x[2] = np.nextafter(np.float16(1.0), np.float16(np.inf))
            elif kind == 2:
                x[2] = np.nextafter(np.float16(1.0), np.float16(-np.inf))
            x *= 2.0 ** ((t % 5) - 2) * (-1.0 if (t + g) % 2 else 1.0)
            out[t, 64 * g:64 * g + 64] = x[rng.permutation(64)]
    return out.astype(np.float16)


def test_prefill_hybrid_choice_on_its_boundary():
    """Inner key groups whose symmetric/asymmetric test holds with equality,
    or misses it by one ulp of one element (where an estimate of the group
    sum cannot decide): the library's codes and parameters equal the
    oracle's bit for bit, and both choices occur."""
    import oracle as O
    from decode_attention_quantize_amd import KVQCache, config_from_workload
    from gpu_harness import HostLayer, unit_body
    from kvq_unpack import unpack_unit
    wl = W.C5.with_(name="hybrid-boundary", B=1, Hq=1, Hkv=1, T=256, steps=1, v_hadamard=False)
    kb, vb = wl.fixed_pairs[0]
    T, D = wl.T, wl.D
    K = _hybrid_boundary_keys(T, D)
    V = _ties_tensor(T, D, vb, 0.125, False, False)
    say("[hybrid] boundary groups")
    cache = KVQCache(config_from_workload(wl), wl.bit_pairs(), device="cuda")
    cache.prefill(0, torch.from_numpy(K).view(1, 1, T, D).cuda(), torch.from_numpy(V).view(1, 1, T, D).cuda())
    torch.cuda.synchronize()
    s_eff, nb, _ = O.state_prefill(T, wl.sinks, wl.window, wl.flush)
    enc = O.encode_unit(O.scheme_for(wl, 0), K.view(np.uint16), V.view(np.uint16), T, s_eff, nb)
    body, lay = unit_body(cache, 0, 0, HostLayer(cache, 0))
    got = unpack_unit(body, lay, kb, vb, nb, True, wl.k_group, wl.v_group, wl.outliers, 0)
    for key in ("kcodes", "kmeta", "vcodes", "vmeta"):
        bad = np.argwhere(got[key] != enc[key])
        assert bad.size == 0, (key, bad[:5].tolist())
    # symmetric groups carry the scale's sign bit; both kinds are present
    sym = [O.hybrid_is_sym(K[t, 64 * g:64 * g + 64].view(np.uint16).copy(), 1, 10)
           for t in range(nb) for g in range(D // 64)]
    assert any(sym) and not all(sym)
    cache.close()


# Codebook levels on a 2^-10 grid: their midpoints are binary16 values
_MID_LEVELS = np.array([0, 129, 266, 408, 541, 679, 838, 1024], np.float64) / 1024


def _midpoint_tensor(T, D, lv):
    """fp16 [T][D] = w - 0.5 with w in [0, 1]: every key group (32 tokens of a
    channel) and value group (32 channels of a token) holds w = 0 and w = 1, so
    min = -0.5 and s = 1 and the quotient (x - min) / s is w itself; the other
    elements are the levels, their midpoints and both 2^-12 neighbours of
    each.  Two columns per row hold +-100, the row's two sparse outliers."""
    mids = (lv[:-1] + lv[1:]) / 2
    pool = np.concatenate([lv, mids, mids - 2.0 ** -12, mids + 2.0 ** -12,
                           np.clip(lv[1:-1] - 2.0 ** -12, 0, 1), np.clip(lv[1:-1] + 2.0 ** -12, 0, 1)])
    t = np.arange(T)[:, None]
    c = np.arange(D)[None, :]
    r = (t + c) % 32
    w = pool[(t * 5 + c * 3) % pool.size]
    w = np.where(r == 0, 0.0, np.where(r == 1, 1.0, w))
    x = w - 0.5
    tt = np.arange(T)
    ca = (2 - tt) % 32 + 32 * (tt % 4)
    cb = (3 - tt) % 32 + 32 * ((tt + 2) % 4)
    x[tt, ca] = 100.0
    x[tt, cb] = -100.0
    assert np.all(x.astype(np.float16).astype(np.float64) == x)
    return x.astype(np.float16)


def test_codebook_codes_next_to_the_midpoints():
    """3-bit codebook keys and values whose quotients sit exactly on a level
    midpoint (a tie, decided below it) or 2^-12 to either side: the
    library's codes, parameters and outliers equal the oracle's bit for bit."""
    import oracle as O
    from decode_attention_quantize_amd import KVQCache, config_from_workload
    from gpu_harness import HostLayer, unit_body
    from kvq_unpack import unpack_unit
    wl = W.C4.with_(name="nuq-midpoints", B=1, Hq=1, Hkv=1, T=256, steps=1)
    T, D = wl.T, wl.D
    cb = np.zeros((1, 2, 8), np.uint16)
    cb[0, 0] = _MID_LEVELS.astype(np.float16).view(np.uint16)
    cb[0, 1] = _MID_LEVELS.astype(np.float16).view(np.uint16)
    K = _midpoint_tensor(T, D, _MID_LEVELS)
    V = np.ascontiguousarray(K[::-1])
    say("[nuq] codes next to the midpoints")
    cache = KVQCache(config_from_workload(wl), wl.bit_pairs(), cb, device="cuda")
    cache.prefill(0, torch.from_numpy(K).view(1, 1, T, D).cuda(), torch.from_numpy(V).view(1, 1, T, D).cuda())
    torch.cuda.synchronize()
    s_eff, nb, _ = O.state_prefill(T, wl.sinks, wl.window, wl.flush)
    sc = O.scheme_for(wl, 0)
    for i in range(8):
        sc.levels_k[i] = int(cb[0, 0, i])
        sc.levels_v[i] = int(cb[0, 1, i])
    enc = O.encode_unit(sc, K.view(np.uint16), V.view(np.uint16), T, s_eff, nb)
    body, lay = unit_body(cache, 0, 0, HostLayer(cache, 0))
    got = unpack_unit(body, lay, 3, 3, nb, False, wl.k_group, wl.v_group, wl.outliers, 0)
    for key in ("kcodes", "kmeta", "vcodes", "vmeta", "kocol", "koval", "vocol", "voval"):
        bad = np.argwhere(got[key] != enc[key])
        assert bad.size == 0, (key, bad[:5].tolist())
    # the construction reaches every code, and the tie elements' quotients are exact
    assert set(np.unique(enc["kcodes"]).tolist()) == set(range(8))
    assert np.all(enc["kmeta"][..., 0] == np.float16(1.0).view(np.uint16))
    cache.close()


@pytest.mark.parametrize("name", ["C1", "C2r", "C3r", "C5r", "C4r", "P5r", "P5r-ternary",
                                  "short-prompt-sinks-then-flush"])
def test_fused_append_decode_matches_the_two_calls(name):
    """kvq_append_decode_attn stands for kvq_append_token + kvq_decode_attn:
    at every step the outputs and the layers' buffers are bit-identical to
    the two calls' (the fused launch where the token only needs storing and
    the layer runs the matrix-core kernel, the two calls otherwise), and the
    fused run passes the oracle checks."""
    from gpu_harness import HostLayer
    wl = REDUCED.get(name) or EDGE[name]
    c0, o0 = run_gpu(wl)
    c1, o1 = run_gpu(wl, fused=True)
    for l in o0:
        for i in o0[l]:
            assert torch.equal(o0[l][i], o1[l][i]), (name, l, i)
        h0, h1 = HostLayer(c0, l), HostLayer(c1, l)
        assert h0.state == h1.state
        assert np.array_equal(h0.body, h1.body) and np.array_equal(h0.fp16, h1.fp16), (name, l)
    worst = 0.0
    for l in range(wl.L):
        worst = max(worst, check_units(wl, c1, o1, l, range(wl.units), label=f"{name}/fused")[0])
    say(f"[fused] {name}: outputs and buffers equal to append + decode; oracle worst {worst:.3e}")
    c0.close()
    c1.close()


def test_unbound_layer_refuses_device_calls():
    from decode_attention_quantize_amd import KVQCache, KVQError, config_from_workload
    wl = W.C1
    cache = KVQCache(config_from_workload(wl), wl.bit_pairs(), device="cuda")
    k = wl.k(0, 0, 1, 0, 1, 0, wl.T, device="cuda").contiguous()
    v = wl.v(0, 0, 1, 0, 1, 0, wl.T, device="cuda").contiguous()
    cache.prefill(0, k, v)
    q = wl.q(0, 0, device="cuda").contiguous()
    cache.decode(0, q)
    cache.unbind(0)
    with pytest.raises(KVQError) as e:
        cache.decode(0, q)
    assert e.value.status == 4
    with pytest.raises(ValueError):
        cache.decode(0, q[:, :, :64].contiguous())           # wrong shape, refused before the call
    with pytest.raises(ValueError):
        cache.decode(0, q.cpu())                              # host tensor
    cache.bind(0)
    cache.prefill(0, k, v)
    with pytest.raises(TypeError):
        cache.decode(0, q, torch.empty(q.shape, dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()
    cache.close()


# ---------------------------------------------------------------- full sizes, every unit
def _full(wl, steps, layers=None):
    """Every unit of the full-size workload against the oracle at the given
    decode steps (codes, parameters and fp16 area bit-exact; outputs within
    the bound)."""
    layers = list(range(wl.L)) if layers is None else layers
    say(f"[parity-full] {wl.name}: {wl.units} units x {len(layers)} layers, steps {sorted(steps)}")
    cache, outs = run_gpu(wl, keep_steps=steps)
    worst = (0.0, -1, -1)
    for l in layers:
        e, u = check_units(wl, cache, outs, l, range(wl.units), check_steps=steps, label=f"{wl.name} l{l}")
        worst = max(worst, (e, l, u))
        say(f"[parity-full] {wl.name} layer {l}: {wl.units} units pass, worst {e:.3e} (unit {u})")
    say(f"[parity-full] {wl.name}: worst row error {worst[0]:.3e} (layer {worst[1]}, unit {worst[2]})")
    cache.close()
    return worst[0]


@pytest.mark.timeout(900)
def test_full_c2_every_unit():
    _full(W.C2, {0, 31, 63})


@pytest.mark.timeout(900)
def test_full_c3_every_unit():
    _full(W.C3, {31, 63})


@pytest.mark.timeout(900)
def test_full_c4_every_unit():
    _full(W.C4, {0, 31})


@pytest.mark.timeout(900)
def test_full_c5_every_unit():
    _full(W.C5, {1, 3})


@pytest.mark.timeout(900)
def test_full_c5_key_norm_every_unit():
    _full(W.C5.with_(k_norm=True), {3})


@pytest.mark.timeout(900)
def test_full_c5_mixed_groups_every_unit():
    _full(W.C5.with_(k_hi_groups=1), {3})


@pytest.mark.timeout(900)
def test_full_c2_hadamard_values_every_unit():
    _full(W.C2.with_(v_hadamard=True), {0, 63})


@pytest.mark.timeout(900)
def test_full_c2_ternary_values_every_unit():
    _full(W.C2.with_(v_ternary=True), {0, 63})


# ---------------------------------------------------------------- calibration on the library's records
def test_library_quantizer_mse_equals_the_calibration_mse():
    """RateQuant's distortion calibration measured on the library itself: a
    Llama-3-8B shaped layer is prefilled at each width the cache implements,
    the packed records are unpacked with the layout of include/kvq.h and
    dequantized with the header's formulas (code * s + z), and the keys' and
    values' MSE equal those of the CPU calibration test."""
    from kvq_unpack import unpack_unit
    from test_rate_calibration import WIDTHS, calibration_mse
    from gpu_harness import unit_body
    units, T = [0, 9, 37], 512
    for bits in WIDTHS:
        wl = W.C3.with_(L=1, T=T, steps=0, fixed_pairs=((bits, bits),))
        cache, _ = run_gpu(wl, steps=0)
        s_eff, nb = cache.state(0)[1], cache.state(0)[2]
        ek = ev = 0.0
        for u in units:
            body, lay = unit_body(cache, 0, u)
            got = unpack_unit(body, lay, bits, bits, nb, False, 32, 32, 0)
            b, h = divmod(u, wl.Hkv)
            kx = wl.k(0, b, b + 1, h, h + 1, 0, T).reshape(T, 128).double().numpy()[s_eff:s_eff + nb]
            vx = wl.v(0, b, b + 1, h, h + 1, 0, T).reshape(T, 128).double().numpy()[s_eff:s_eff + nb]
            ks = np.repeat(got["kmeta"][:, :, 0].view(np.float16).astype(np.float64), 32, axis=0)
            kz = np.repeat(got["kmeta"][:, :, 1].view(np.float16).astype(np.float64), 32, axis=0)
            vs = np.repeat(got["vmeta"][:, :, 0].view(np.float16).astype(np.float64), 32, axis=1)
            vz = np.repeat(got["vmeta"][:, :, 1].view(np.float16).astype(np.float64), 32, axis=1)
            kh = got["kcodes"].astype(np.float64) * ks + kz
            vh = got["vcodes"].astype(np.float64) * vs + vz
            ek += float(np.mean((kh - kx) ** 2))
            ev += float(np.mean((vh - vx) ** 2))
        ek, ev = ek / len(units), ev / len(units)
        ok, ov = calibration_mse(W.C3, 0, units, T, bits)
        say(f"[calibration] {bits}-bit: library mse K {ek:.6e} V {ev:.6e}")
        assert np.isclose(ek, ok, rtol=1e-12, atol=0) and np.isclose(ev, ov, rtol=1e-12, atol=0), (bits, ek, ok, ev, ov)
        cache.close()
