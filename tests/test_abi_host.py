"""Host-side checks of the C ABI (no GPU needed).

The library is loaded and every symbol include/kvq.h declares must be
exported; configuration validation, buffer sizing and the call-order / capacity
errors are all decided on the host before any launch, so they run here with
dummy (never dereferenced) aligned pointers.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

from decode_attention_quantize_amd import build as kb
from decode_attention_quantize_amd import kvq as K
from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built():
    if kb.is_stale():
        kb.build()
    K.lib()


def header_functions():
    txt = open(os.path.join(ROOT, "include", "kvq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:kvq_status|const char\*)\s+(kvq_\w+)\s*\(", txt, re.M)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) == len(K.EXPORTS), names
    L = C.CDLL(K.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(K.EXPORTS)


def test_status_strings():
    for s in range(6):
        assert K.status_str(s)
    assert K.status_str(99) == "unknown status"


def _cfg(**kw):
    base = dict(B=1, Hq=4, Hkv=2, L=2, max_tokens=1000)
    base.update(kw)
    return K.make_config(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), K.KVQ_ERR_ARG),
    (dict(Hq=3, Hkv=2), K.KVQ_ERR_ARG),
    (dict(max_tokens=0), K.KVQ_ERR_ARG),
    (dict(D=64), K.KVQ_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=2), K.KVQ_ERR_UNSUPPORTED),       # 3 q heads per kv head
    (dict(Hq=64, Hkv=2), K.KVQ_ERR_UNSUPPORTED),      # 32 rows per kv head
    (dict(k_group=16), K.KVQ_ERR_UNSUPPORTED),        # per-channel groups must be 32 tokens
    (dict(k_mode=1, k_group=128), K.KVQ_ERR_UNSUPPORTED),
    (dict(v_group=128), K.KVQ_ERR_UNSUPPORTED),
    (dict(k_mode=7), K.KVQ_ERR_ARG),
    (dict(outliers=9), K.KVQ_ERR_ARG),
    (dict(k_pre_rope=1, rope_base=0.0), K.KVQ_ERR_ARG),
    (dict(k_norm=2, k_mode=1, k_group=64), K.KVQ_ERR_ARG),
    (dict(k_norm=1), K.KVQ_ERR_UNSUPPORTED),          # normalization is for inner key groups
    (dict(v_mode=3), K.KVQ_ERR_ARG),
    (dict(k_hi_groups=-1, k_mode=1, k_group=64), K.KVQ_ERR_ARG),
    (dict(k_hi_groups=1), K.KVQ_ERR_UNSUPPORTED),     # mixed widths are for inner key groups
    (dict(k_hi_groups=3, k_mode=1, k_group=64), K.KVQ_ERR_ARG),  # a token has two groups of 64
    (dict(k_hi_groups=1, k_mode=1, k_group=64, outliers=2), K.KVQ_ERR_UNSUPPORTED),
])
def test_create_rejects(kw, status):
    with pytest.raises(K.KVQError) as e:
        K.kvq_create(_cfg(**kw), [(4, 4), (4, 2)])
    assert e.value.status == status


def test_create_rejects_bits_and_codebooks():
    with pytest.raises(K.KVQError) as e:
        K.kvq_create(_cfg(), [(4, 5), (4, 2)])
    assert e.value.status == K.KVQ_ERR_UNSUPPORTED
    with pytest.raises(K.KVQError) as e:
        K.kvq_create(_cfg(nuq=1), [(3, 3), (3, 3)])      # codebooks missing
    assert e.value.status == K.KVQ_ERR_ARG
    cb = np.zeros((2, 2, 8), np.uint16)
    with pytest.raises(K.KVQError) as e:
        K.kvq_create(_cfg(nuq=1), [(4, 4), (3, 3)], cb)  # codebook mode is 3-bit
    assert e.value.status == K.KVQ_ERR_UNSUPPORTED
    cb[1, 0, 3] = 0x7C00
    with pytest.raises(K.KVQError) as e:
        K.kvq_create(_cfg(nuq=1), [(3, 3), (3, 3)], cb)  # infinite level
    assert e.value.status == K.KVQ_ERR_ARG
    with pytest.raises(K.KVQError) as e:
        K.kvq_create(_cfg(v_mode=K.KVQ_V_TERNARY), [(4, 2), (4, 4)])  # ternary values are 2-bit codes
    assert e.value.status == K.KVQ_ERR_UNSUPPORTED
    with pytest.raises(K.KVQError) as e:
        K.kvq_create(_cfg(v_mode=K.KVQ_V_TERNARY, nuq=1), [(3, 3), (3, 3)], cb)
    assert e.value.status == K.KVQ_ERR_UNSUPPORTED
    rc = K.lib().kvq_create(None, None, None, None)
    assert rc == K.KVQ_ERR_ARG


def _expected_record(kb_, vb, k_inner=False, kg=32, vg=32, outk=0, k_hi=0):
    a16 = lambda x: (x + 15) // 16 * 16
    kc = 32 * 128 * kb_ // 8
    km = 32 * (128 // kg) * 4 if k_inner else 512
    vc = 32 * 128 * vb // 8
    vm = 2 * (128 // vg) * 32 * 2
    ko = 32 * outk * 4
    m = k_hi if (k_inner and kb_ == 4) else 0
    kx = 32 * m * kg // 2                     # low nibbles of the 8-bit groups
    ks = 32 if m else 0                       # per-token group masks
    off = [0]
    for sz in (kc, km, vc, vm, ko, ko, kx, ks):
        off.append(a16(off[-1] + sz))
    return off[:8], (off[8] + 127) // 128 * 128


VARIANTS = {"C5n": dict(k_norm=True), "C5m": dict(k_hi_groups=1),
            "C5m32": dict(k_group=32, k_hi_groups=2, fixed_pairs=((4, 2),))}


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5", "C5n", "C5m", "C5m32"])
def test_layout_and_sizes_follow_the_spec(name):
    wl = W.ALL[name] if name in W.ALL else W.C5.with_(**VARIANTS[name])
    h = K.kvq_create(K.config_from_workload(wl), wl.bit_pairs(), wl.codebooks())
    try:
        pairs = wl.bit_pairs()
        units = wl.B * wl.Hkv
        max_tokens = wl.T + (wl.steps if wl.append else 0)
        for l in range(min(wl.L, 6)):
            kb_, vb = pairs[l]
            lay = K.kvq_block_layout(h, l)
            offs, rec = _expected_record(kb_, vb, wl.k_mode == "inner", wl.k_group, wl.v_group, wl.outliers,
                                         wl.k_hi_groups)
            assert [lay[k] for k in ("k_codes", "k_meta", "v_codes", "v_meta", "k_out", "v_out",
                                     "k_ext", "k_sel")] == offs
            assert lay["record_bytes"] == rec
            assert lay["k_row_bytes"] == 128 * kb_ // 8
            F = 32 if wl.k_mode == "channel" else 1
            assert lay["flush_tokens"] == F
            wcap = -(-(wl.window + F) // 32) * 32
            scap = -(-wl.sinks // 32) * 32
            assert lay["window_cap"] == wcap and lay["sink_cap"] == scap
            sizes = K.kvq_layer_buffer_sizes(h, l)
            assert sizes[0] == units * (-(-max_tokens // 32)) * rec
            assert sizes[1] == units * 2 * (scap + wcap) * 128 * 2 + (units * 128 if wl.k_norm else 0)
        assert K.kvq_workspace_size(h) > 0
    finally:
        K.kvq_destroy(h)


def test_average_bits_from_code_bytes():
    """f_m(P) = sum(P)/2L (KVTuner review, method step 0) equals the mean bit
    width implied by the packed code bytes of each layer's records."""
    wl = W.C3
    h = K.kvq_create(K.config_from_workload(wl), wl.bit_pairs())
    try:
        bits = []
        for l in range(wl.L):
            lay = K.kvq_block_layout(h, l)
            k_bits = (lay["k_meta"] - lay["k_codes"]) * 8 / (32 * 128)
            v_bits = (lay["v_meta"] - lay["v_codes"]) * 8 / (32 * 128)
            bits += [k_bits, v_bits]
        pairs = wl.bit_pairs()
        f_m = sum(kb_ + vb for kb_, vb in pairs) / (2 * wl.L)
        assert np.mean(bits) == f_m
        assert set(pairs) <= set(W.PAIR_SET) and len(set(pairs)) == 5
        code, stored = K.kvq_average_bits(h)
        assert code == f_m
        recs = [K.kvq_block_layout(h, l)["record_bytes"] for l in range(wl.L)]
        assert stored == np.mean([8 * r / (2 * 32 * 128) for r in recs]) and stored > code
    finally:
        K.kvq_destroy(h)


@pytest.mark.parametrize("kg,m,pairs,f_m", [
    (64, 1, [(4, 2), (8, 8)], (6 + 2 + 8 + 8) / 4),    # one of two groups at 8 bits: keys 6 bits
    (32, 1, [(4, 4)], (5 + 4) / 2),                    # one of four: 5 bits
    (32, 3, [(4, 2), (2, 2)], (7 + 2 + 2 + 2) / 4),    # three of four: 7; the 2-bit layer unchanged
    (64, 0, [(4, 2)], 3.0),
])
def test_average_bits_counts_mixed_groups(kg, m, pairs, f_m):
    # f_m = sum(P)/2L with a mixed layer's key width averaged over its groups
    cfg = K.make_config(1, 8, 8, len(pairs), 64, k_mode=K.KVQ_K_INNER, k_group=kg, k_hybrid=1,
                        k_hi_groups=m)
    h = K.kvq_create(cfg, pairs)
    try:
        assert K.kvq_average_bits(h)[0] == f_m
    finally:
        K.kvq_destroy(h)


def test_call_order_and_capacity_errors_on_host():
    cfg = _cfg(max_tokens=100, window=8)
    h = K.kvq_create(cfg, [(4, 4), (4, 2)])
    fake = 1 << 20                      # aligned, never dereferenced: every call fails first
    stream = None
    try:
        def st(fn, *a):
            return fn(*a)
        L = K.lib()
        assert L.kvq_quantize_prefill(h, 0, fake, fake, 10, None, stream) == K.KVQ_ERR_STATE   # unbound
        assert L.kvq_decode_attn(h, 0, fake, fake, fake, stream) == K.KVQ_ERR_STATE
        assert L.kvq_append_token(h, 0, fake, fake, stream) == K.KVQ_ERR_STATE
        assert L.kvq_append_decode_attn(h, 0, fake, fake, fake, fake, fake, stream) == K.KVQ_ERR_STATE
        assert L.kvq_quantize_prefill(h, 5, fake, fake, 10, None, stream) == K.KVQ_ERR_ARG     # layer
        arr = (C.c_void_p * 2)(fake, fake + 1)                                                # misaligned
        assert L.kvq_bind_layer(h, 0, arr) == K.KVQ_ERR_ARG
        arr = (C.c_void_p * 2)(fake, fake)
        assert L.kvq_bind_layer(h, 0, arr) == K.KVQ_OK
        assert L.kvq_quantize_prefill(h, 0, fake, fake, 101, None, stream) == K.KVQ_ERR_CAPACITY
        assert L.kvq_quantize_prefill(h, 0, fake, fake, -1, None, stream) == K.KVQ_ERR_ARG
        assert L.kvq_quantize_prefill(h, 0, None, fake, 4, None, stream) == K.KVQ_ERR_ARG
        assert L.kvq_append_token(h, 0, fake, fake, stream) == K.KVQ_ERR_STATE               # before prefill
        assert L.kvq_decode_attn(h, 0, fake, fake, fake, stream) == K.KVQ_ERR_STATE
        assert L.kvq_decode_attn(h, 0, None, fake, fake, stream) == K.KVQ_ERR_ARG
        assert L.kvq_append_decode_attn(h, 0, fake, fake, fake, fake, fake, stream) == K.KVQ_ERR_STATE
        for i in range(5):                      # every pointer but the stream is required
            args = [fake] * 5
            args[i] = None
            assert L.kvq_append_decode_attn(h, 0, *args, stream) == K.KVQ_ERR_ARG, i
        assert K.kvq_layer_state(h, 0) == (0, 0, 0, 0)
        assert L.kvq_layer_state(h, 9, None, None, None, None) == K.KVQ_ERR_ARG
        # an unbound layer refuses device work again until it is bound
        assert L.kvq_unbind_layer(h, 0) == K.KVQ_OK
        assert L.kvq_quantize_prefill(h, 0, fake, fake, 10, None, stream) == K.KVQ_ERR_STATE
        assert L.kvq_unbind_layer(h, 7) == K.KVQ_ERR_ARG
        assert L.kvq_decode_nonfinite_rows(h, None, stream, None) == K.KVQ_ERR_ARG
    finally:
        K.kvq_destroy(h)
    assert K.lib().kvq_destroy(None) == K.KVQ_OK
