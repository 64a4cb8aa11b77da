"""ctypes front end of the C++ oracle (kvq_oracle.cpp) plus a per-unit driver.

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "kvq_oracle.cpp")
SO = os.path.join(_HERE, "liboracle.so")
CXXFLAGS = ["-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (plain C++17, no contraction, no fast-math)."""
    if force or not os.path.exists(SO) or os.path.getmtime(SO) < os.path.getmtime(SRC):
        tmp = SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", *CXXFLAGS, SRC, "-o", tmp])
        os.replace(tmp, SO)
    return SO


class OScheme(C.Structure):
    _fields_ = [
        ("D", C.c_int32), ("k_mode", C.c_int32), ("k_group", C.c_int32), ("v_group", C.c_int32),
        ("k_bits", C.c_int32), ("v_bits", C.c_int32), ("k_hybrid", C.c_int32),
        ("ratio_num", C.c_int32), ("ratio_den", C.c_int32), ("nuq", C.c_int32),
        ("outliers", C.c_int32), ("v_hadamard", C.c_int32), ("pre_rope", C.c_int32),
        ("rope_base", C.c_double), ("levels_k", C.c_uint16 * 8), ("levels_v", C.c_uint16 * 8),
        ("v_ternary", C.c_int32), ("k_hi_groups", C.c_int32),
    ]


def _p(a, t):
    return a.ctypes.data_as(C.POINTER(t)) if a is not None else None


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            L = C.CDLL(SO)
            u16p, u8p, i32p, f64p = (C.POINTER(C.c_uint16), C.POINTER(C.c_uint8),
                                     C.POINTER(C.c_int32), C.POINTER(C.c_double))
            L.oq_f64_to_f16.restype = C.c_uint16
            L.oq_f64_to_f16.argtypes = [C.c_double]
            L.oq_f16_to_f64.restype = C.c_double
            L.oq_f16_to_f64.argtypes = [C.c_uint16]
            L.oq_f64_to_f16_n.argtypes = [f64p, u16p, C.c_int64]
            L.oq_f32_to_f16_n.argtypes = [C.POINTER(C.c_float), u16p, C.c_int64]
            L.oq_quant_asym.argtypes = [u16p, u8p, C.c_int32, C.c_int32, u8p, u16p]
            L.oq_quant_sym.argtypes = [u16p, C.c_int32, C.c_int32, u8p, u16p]
            L.oq_hybrid_is_sym.argtypes = [u16p, C.c_int32, C.c_int32, C.c_int32]
            L.oq_hybrid_is_sym.restype = C.c_int32
            L.oq_quant_nuq.argtypes = [u16p, u8p, C.c_int32, u16p, u8p, u16p]
            L.oq_quant_tern.argtypes = [u16p, u8p, C.c_int32, u8p, u16p]
            L.oq_topk.argtypes = [u16p, C.c_int32, C.c_int32, i32p]
            L.oq_hadamard_fp16.argtypes = [u16p, C.c_int32, u16p]
            L.oq_hadamard_f64.argtypes = [f64p, C.c_int32, f64p]
            L.oq_dequant.argtypes = [C.c_uint8, C.c_uint16, C.c_uint16, C.c_int32, u16p]
            L.oq_dequant.restype = C.c_double
            L.oq_state_prefill.argtypes = [C.c_int32] * 4 + [i32p] * 3
            L.oq_state_append.argtypes = [i32p, i32p, i32p, i32p, C.c_int32, C.c_int32, C.c_int32]
            L.oq_state_append.restype = C.c_int32
            L.oq_encode_unit.argtypes = [C.POINTER(OScheme), u16p, u16p, C.c_int32, C.c_int32,
                                         C.c_int32, u16p, u8p, u16p, u8p, u16p, i32p, u16p, i32p, u16p,
                                         u8p]
            L.oq_encode_unit.restype = C.c_int32
            L.oq_dequant_unit.argtypes = [C.POINTER(OScheme), u16p, u16p, C.c_int32, C.c_int32,
                                          C.c_int32, C.c_int32, C.c_int32, u8p, u16p, u8p, u16p,
                                          i32p, u16p, i32p, u16p, C.POINTER(C.c_int8), u8p, f64p, f64p]
            L.oq_dequant_unit.restype = C.c_int32
            L.oq_knorm_shifts.argtypes = [u16p, C.c_int32, C.c_int32, C.POINTER(C.c_int8)]
            L.oq_knorm_apply.argtypes = [u16p, C.c_int32, C.c_int32, C.POINTER(C.c_int8), u16p]
            L.oq_attention.argtypes = [f64p, C.c_int32, f64p, f64p, C.c_int32, C.c_int32, C.c_int32, f64p]
            L.oq_attention_split.argtypes = [f64p, C.c_int32, f64p, f64p, C.c_int32, C.c_int32,
                                             C.c_int32, C.c_int32, f64p]
            _lib = L
    return _lib


# ---------------------------------------------------------------- scalar / group helpers
def f64_to_f16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64).ravel()
    out = np.empty(x.size, dtype=np.uint16)
    lib().oq_f64_to_f16_n(_p(x, C.c_double), _p(out, C.c_uint16), x.size)
    return out


def f32_to_f16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(x.size, dtype=np.uint16)
    lib().oq_f32_to_f16_n(_p(x, C.c_float), _p(out, C.c_uint16), x.size)
    return out


def f16_to_f64(h) -> np.ndarray:
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)


def quant_asym(x16, bits, excl=None):
    x16 = np.ascontiguousarray(x16, dtype=np.uint16)
    ex = None if excl is None else np.ascontiguousarray(excl, dtype=np.uint8)
    codes = np.empty(x16.size, np.uint8)
    meta = np.empty(2, np.uint16)
    lib().oq_quant_asym(_p(x16, C.c_uint16), _p(ex, C.c_uint8), x16.size, bits,
                        _p(codes, C.c_uint8), _p(meta, C.c_uint16))
    return codes, meta


def quant_sym(x16, bits):
    x16 = np.ascontiguousarray(x16, dtype=np.uint16)
    codes = np.empty(x16.size, np.uint8)
    meta = np.empty(2, np.uint16)
    lib().oq_quant_sym(_p(x16, C.c_uint16), x16.size, bits, _p(codes, C.c_uint8), _p(meta, C.c_uint16))
    return codes, meta


def hybrid_is_sym(x16, num=1, den=10) -> bool:
    x16 = np.ascontiguousarray(x16, dtype=np.uint16)
    return bool(lib().oq_hybrid_is_sym(_p(x16, C.c_uint16), x16.size, num, den))


def quant_tern(x16, excl=None):
    """Ternary levels {-s, 0, s} in 2-bit codes: (codes, [s, z])."""
    x16 = np.ascontiguousarray(x16, dtype=np.uint16)
    ex = None if excl is None else np.ascontiguousarray(excl, dtype=np.uint8)
    codes = np.empty(x16.size, np.uint8)
    meta = np.empty(2, np.uint16)
    lib().oq_quant_tern(_p(x16, C.c_uint16), _p(ex, C.c_uint8), x16.size, _p(codes, C.c_uint8),
                        _p(meta, C.c_uint16))
    return codes, meta


def quant_nuq(x16, levels16, excl=None):
    x16 = np.ascontiguousarray(x16, dtype=np.uint16)
    lv = np.ascontiguousarray(levels16, dtype=np.uint16)
    ex = None if excl is None else np.ascontiguousarray(excl, dtype=np.uint8)
    codes = np.empty(x16.size, np.uint8)
    meta = np.empty(2, np.uint16)
    lib().oq_quant_nuq(_p(x16, C.c_uint16), _p(ex, C.c_uint8), x16.size, _p(lv, C.c_uint16),
                       _p(codes, C.c_uint8), _p(meta, C.c_uint16))
    return codes, meta


def topk(row16, k):
    row16 = np.ascontiguousarray(row16, dtype=np.uint16)
    cols = np.empty(k, np.int32)
    lib().oq_topk(_p(row16, C.c_uint16), row16.size, k, _p(cols, C.c_int32))
    return cols


def hadamard_fp16(v16):
    v16 = np.ascontiguousarray(v16, dtype=np.uint16)
    out = np.empty_like(v16)
    lib().oq_hadamard_fp16(_p(v16, C.c_uint16), v16.size, _p(out, C.c_uint16))
    return out


def hadamard_f64(v):
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(v)
    lib().oq_hadamard_f64(_p(v, C.c_double), v.size, _p(out, C.c_double))
    return out


def dequant(code, s16, z16, bits, levels16=None) -> float:
    lv = None if levels16 is None else np.ascontiguousarray(levels16, dtype=np.uint16)
    return lib().oq_dequant(int(code), int(s16), int(z16), bits, _p(lv, C.c_uint16))


# ---------------------------------------------------------------- state machine
def state_prefill(n, S, W, F):
    a, b, c = C.c_int32(), C.c_int32(), C.c_int32()
    lib().oq_state_prefill(n, S, W, F, C.byref(a), C.byref(b), C.byref(c))
    return a.value, b.value, c.value


def state_append(n, s_eff, nb, r, S, W, F):
    """One appended token: (n, s_eff, nb, r, flushed)."""
    a, se, b, c = C.c_int32(n), C.c_int32(s_eff), C.c_int32(nb), C.c_int32(r)
    f = lib().oq_state_append(C.byref(a), C.byref(se), C.byref(b), C.byref(c), S, W, F)
    return a.value, se.value, b.value, c.value, bool(f)


# ---------------------------------------------------------------- unit level
def make_scheme(D=128, k_mode=0, k_group=32, v_group=32, k_bits=4, v_bits=4, k_hybrid=0,
                ratio=(1, 10), nuq=0, outliers=0, v_hadamard=0, pre_rope=0, rope_base=10000.0,
                levels_k=None, levels_v=None, v_ternary=0, k_hi_groups=0) -> OScheme:
    s = OScheme()
    s.D, s.k_mode, s.k_group, s.v_group = D, k_mode, k_group, v_group
    s.k_bits, s.v_bits, s.k_hybrid = k_bits, v_bits, k_hybrid
    s.ratio_num, s.ratio_den = ratio
    s.nuq, s.outliers, s.v_hadamard, s.pre_rope = nuq, outliers, v_hadamard, pre_rope
    s.rope_base = rope_base
    s.v_ternary = v_ternary
    s.k_hi_groups = k_hi_groups
    for i in range(8):
        s.levels_k[i] = int(levels_k[i]) if levels_k is not None else 0
        s.levels_v[i] = int(levels_v[i]) if levels_v is not None else 0
    return s


def scheme_for(wl, layer: int) -> OScheme:
    kb, vb = wl.bit_pairs()[layer]
    cb = wl.codebooks()
    ratio = _ratio(wl.sym_ratio)
    return make_scheme(
        D=wl.D, k_mode=0 if wl.k_mode == "channel" else 1, k_group=wl.k_group, v_group=wl.v_group,
        k_bits=kb, v_bits=vb, k_hybrid=int(wl.k_hybrid), ratio=ratio, nuq=int(wl.nuq),
        outliers=wl.outliers, v_hadamard=int(wl.v_hadamard), pre_rope=int(wl.pre_rope),
        rope_base=wl.rope_base,
        levels_k=None if cb is None else cb[layer, 0], levels_v=None if cb is None else cb[layer, 1],
        v_ternary=int(getattr(wl, "v_ternary", False)),
        k_hi_groups=getattr(wl, "k_hi_groups", 0) if (wl.k_mode == "inner" and kb == 4) else 0)


def _ratio(r: float):
    from fractions import Fraction
    f = Fraction(r).limit_denominator(1000)
    return (f.numerator, f.denominator)


def encode_unit(sc: OScheme, K16, V16, n, s_eff, nb):
    D = sc.D
    K16 = np.ascontiguousarray(K16, dtype=np.uint16).reshape(-1, D)
    V16 = np.ascontiguousarray(V16, dtype=np.uint16).reshape(-1, D)
    assert K16.shape[0] >= n and V16.shape[0] >= n
    ko = max(sc.outliers, 1)
    e = dict(
        vrot=np.empty((n, D), np.uint16),
        kcodes=np.zeros((nb, D), np.uint8),
        kmeta=np.zeros(((nb // sc.k_group) if sc.k_mode == 0 else nb,
                        D if sc.k_mode == 0 else D // sc.k_group, 2), np.uint16),
        vcodes=np.zeros((nb, D), np.uint8),
        vmeta=np.zeros((nb, D // sc.v_group, 2), np.uint16),
        kocol=np.zeros((nb, ko), np.int32), koval=np.zeros((nb, ko), np.uint16),
        vocol=np.zeros((nb, ko), np.int32), voval=np.zeros((nb, ko), np.uint16),
    )
    if sc.k_mode == 1:
        e["kwidth"] = np.zeros((nb, D // sc.k_group), np.uint8)
    rc = lib().oq_encode_unit(C.byref(sc), _p(K16, C.c_uint16), _p(V16, C.c_uint16), n, s_eff, nb,
                              _p(e["vrot"], C.c_uint16), _p(e["kcodes"], C.c_uint8),
                              _p(e["kmeta"], C.c_uint16), _p(e["vcodes"], C.c_uint8),
                              _p(e["vmeta"], C.c_uint16), _p(e["kocol"], C.c_int32),
                              _p(e["koval"], C.c_uint16), _p(e["vocol"], C.c_int32),
                              _p(e["voval"], C.c_uint16), _p(e.get("kwidth"), C.c_uint8))
    if rc != 0:
        raise ValueError("oracle: unsupported scheme")
    if sc.outliers == 0:
        for k in ("kocol", "koval", "vocol", "voval"):
            e[k] = e[k][:, :0]
    return e


def knorm_shifts(K16_prefill) -> np.ndarray:
    """int8 [D] per-channel key normalization shifts from the prefill rows."""
    K16 = np.ascontiguousarray(K16_prefill, dtype=np.uint16)
    T, D = K16.shape
    out = np.zeros(D, np.int8)
    lib().oq_knorm_shifts(_p(K16, C.c_uint16), T, D, _p(out, C.c_int8))
    return out


def knorm_apply(K16, shift) -> np.ndarray:
    """uint16 [n][D] normalized keys fp16(K * 2^shift) (saturating)."""
    K16 = np.ascontiguousarray(K16, dtype=np.uint16)
    n, D = K16.shape
    out = np.empty((n, D), np.uint16)
    sh = np.ascontiguousarray(shift, dtype=np.int8)
    lib().oq_knorm_apply(_p(K16, C.c_uint16), n, D, _p(sh, C.c_int8), _p(out, C.c_uint16))
    return out


def dequant_unit(sc: OScheme, K16, enc, n, s_eff, nb, t_begin=0, t_end=None, Khat=None, Vhat=None,
                 kshift=None):
    """binary64 K-hat, V-hat [n][D] (rows t_begin..t_end rebuilt).  kshift: key
    normalization shifts of the unit (body keys are scaled back by 2^-shift)."""
    D = sc.D
    t_end = n if t_end is None else t_end
    K16 = np.ascontiguousarray(K16, dtype=np.uint16).reshape(-1, D)
    if Khat is None:
        Khat = np.zeros((n, D), np.float64)
        Vhat = np.zeros((n, D), np.float64)
    ko = max(sc.outliers, 1)
    def pad(a, dt):
        return np.ascontiguousarray(a if a.shape[1] else np.zeros((max(a.shape[0], 1), ko), dt))
    kocol, koval = pad(enc["kocol"], np.int32), pad(enc["koval"], np.uint16)
    vocol, voval = pad(enc["vocol"], np.int32), pad(enc["voval"], np.uint16)
    rc = lib().oq_dequant_unit(C.byref(sc), _p(K16, C.c_uint16), _p(enc["vrot"], C.c_uint16), n,
                               s_eff, nb, t_begin, t_end, _p(enc["kcodes"], C.c_uint8),
                               _p(enc["kmeta"], C.c_uint16), _p(enc["vcodes"], C.c_uint8),
                               _p(enc["vmeta"], C.c_uint16), _p(kocol, C.c_int32),
                               _p(koval, C.c_uint16), _p(vocol, C.c_int32), _p(voval, C.c_uint16),
                               _p(None if kshift is None else np.ascontiguousarray(kshift, dtype=np.int8),
                                  C.c_int8),
                               _p(enc.get("kwidth"), C.c_uint8),
                               _p(Khat, C.c_double), _p(Vhat, C.c_double))
    assert rc == 0
    return Khat, Vhat


def attention(q, Khat, Vhat, unrotate=False):
    q = np.ascontiguousarray(q, dtype=np.float64)
    G, D = q.shape
    n = Khat.shape[0]
    out = np.empty((G, D), np.float64)
    lib().oq_attention(_p(q, C.c_double), G, _p(np.ascontiguousarray(Khat), C.c_double),
                       _p(np.ascontiguousarray(Vhat), C.c_double), n, D, int(unrotate),
                       _p(out, C.c_double))
    return out


def attention_split(q, Khat, Vhat, nsplit, unrotate=False):
    q = np.ascontiguousarray(q, dtype=np.float64)
    G, D = q.shape
    n = Khat.shape[0]
    out = np.empty((G, D), np.float64)
    lib().oq_attention_split(_p(q, C.c_double), G, _p(np.ascontiguousarray(Khat), C.c_double),
                             _p(np.ascontiguousarray(Vhat), C.c_double), n, D, int(unrotate),
                             nsplit, _p(out, C.c_double))
    return out


def unit_inputs(wl, layer, b, h, n_total):
    """uint16 [n_total][D] K and V of one (batch, kv-head) unit (synthetic)."""
    K = wl.k(layer, b, b + 1, h, h + 1, 0, n_total).reshape(n_total, wl.D)
    V = wl.v(layer, b, b + 1, h, h + 1, 0, n_total).reshape(n_total, wl.D)
    return K.numpy().view(np.uint16), V.numpy().view(np.uint16)


def run_unit(wl, layer, b, h, steps=None, only_steps=None):
    """Oracle for one unit through prefill and the decode steps.

    Returns dict(states=[(n, s_eff, nb, r)], out={step: [Gq][D] float64}, enc=final
    encoding, s_eff, n_final, nb_final).  The body encoding at any step is a
    prefix of the final one (blocks are pure functions of their tokens), so the
    cache is encoded once and each step dequantizes its own prefix.
    """
    steps = wl.steps if steps is None else steps
    sc = scheme_for(wl, layer)
    F = wl.flush
    n_total = wl.T + (steps if wl.append else 0)
    K, V = unit_inputs(wl, layer, b, h, n_total)
    s_eff, nb, r = state_prefill(wl.T, wl.sinks, wl.window, F)
    n = wl.T
    states = []
    for i in range(steps):
        if wl.append:
            n, s_eff, nb, r, _ = state_append(n, s_eff, nb, r, wl.sinks, wl.window, F)
        states.append((n, s_eff, nb, r))
    nb_final = states[-1][2] if states else nb
    n_final = states[-1][0] if states else n
    kshift = None
    Kq = K
    if getattr(wl, "k_norm", False):
        # InnerQ method 4: shifts from the prefill rows, body keys quantized
        # in the normalized domain, fp16 sink/window rows kept as given
        kshift = knorm_shifts(K[:wl.T])
        Kq = knorm_apply(K, kshift)
    enc = encode_unit(sc, Kq, V, n_final, s_eff, nb_final)
    Kf, Vf = dequant_unit(sc, K, enc, n_final, s_eff, nb_final, kshift=kshift)
    gq = wl.gq
    outs = {}
    for i, (n_i, se_i, nb_i, r_i) in enumerate(states):
        if only_steps is not None and i not in only_steps:
            continue
        Kh, Vh = Kf[:n_i].copy(), Vf[:n_i].copy()
        lo = se_i + nb_i
        if lo < n_i:
            dequant_unit(sc, K, enc, n_i, se_i, nb_i, lo, n_i, Kh, Vh, kshift=kshift)
        q = wl.q(layer, i, b0=b, b1=b + 1, h0=h * gq, h1=(h + 1) * gq).reshape(gq, wl.D)
        outs[i] = attention(q.double().numpy(), Kh, Vh, unrotate=bool(wl.v_hadamard))
    return dict(states=states, out=outs, enc=enc, s_eff=s_eff, n_final=n_final,
                nb_final=nb_final, K=K, V=V, scheme=sc, kshift=kshift)
