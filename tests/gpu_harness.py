"""Drive a workload through the GPU library and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O
from decode_attention_quantize_amd import KVQCache, config_from_workload
from kvq_unpack import unpack_unit

TOL = 2e-3   # row-max-normalised error bound on attention outputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(wl, layers=None, steps=None, keep_units=None, device="cuda", fill=None, keep_steps=None,
            fused=False):
    """Prefill every layer, then per step: per layer append (when the workload
    appends) and decode -- as one kvq_append_decode_attn call when fused.
    Returns outputs [layer][step] -> cpu fp32 [B][Hq][D] (only for the kept
    units when keep_units is given; only the kept steps when keep_steps is
    given).  fill: byte the layer buffers hold before the prefill (default
    zeros)."""
    dev = torch.device(device)
    layers = list(range(wl.L)) if layers is None else layers
    steps = wl.steps if steps is None else steps
    cache = KVQCache(config_from_workload(wl), wl.bit_pairs(), wl.codebooks(), device=dev,
                     layers=layers, fill=fill)
    B, Hkv, Hq, T = wl.B, wl.Hkv, wl.Hq, wl.T
    for l in layers:
        k = wl.k(l, 0, B, 0, Hkv, 0, T, device=dev).contiguous()
        v = wl.v(l, 0, B, 0, Hkv, 0, T, device=dev).contiguous()
        cache.prefill(l, k, v)
        del k, v
    outs = {l: {} for l in layers}
    for i in range(steps):
        for l in layers:
            q = wl.q(l, i, device=dev).contiguous()
            if wl.append:
                kt = wl.k(l, 0, B, 0, Hkv, T + i, T + i + 1, device=dev).reshape(B, Hkv, wl.D).contiguous()
                vt = wl.v(l, 0, B, 0, Hkv, T + i, T + i + 1, device=dev).reshape(B, Hkv, wl.D).contiguous()
                if fused:
                    o = cache.append_decode(l, kt, vt, q)
                else:
                    cache.append(l, kt, vt)
                    o = cache.decode(l, q)
            else:
                o = cache.decode(l, q)
            if keep_steps is not None and i not in keep_steps:
                continue
            if keep_units is None:
                outs[l][i] = o.cpu()
            else:
                outs[l][i] = {u: o[u // Hkv, (u % Hkv) * wl.gq:(u % Hkv + 1) * wl.gq].cpu()
                              for u in keep_units}
    torch.cuda.synchronize()
    return cache, outs


class HostLayer:
    """Host copies of one layer's two device buffers and its state, taken
    once so that many units can be checked from threads without GPU calls."""

    def __init__(self, cache, layer):
        self.lay = cache.layout(layer)
        self.body = cache.raw(layer, 0).cpu().numpy()
        self.fp16 = cache.raw(layer, 1).cpu().numpy()
        self.state = cache.state(layer)
        self.units = cache.cfg.batch * cache.cfg.n_kv_heads


def _host(cache, layer, host):
    return host if host is not None else HostLayer(cache, layer)


def unit_body(cache, layer, u, host=None):
    h = _host(cache, layer, host)
    per_unit = h.body.size // h.units
    return h.body[u * per_unit:(u + 1) * per_unit], h.lay


def unit_fp16(cache, layer, u, scap, wcap, host=None):
    """(K, V) of one unit's fp16 area as [slots][128] arrays, from the
    documented layout: keys token-major, values 8-slot interleaved."""
    h = _host(cache, layer, host)
    slots = scap + wcap
    per = 2 * slots * 128 * 2
    raw = h.fp16[u * per:(u + 1) * per].view(np.uint16)
    k = raw[:slots * 128].reshape(slots, 128)
    v = raw[slots * 128:].reshape(slots // 8, 128, 8).transpose(0, 2, 1).reshape(slots, 128)
    return k, v


def unit_kshift(cache, layer, u, scap, wcap, host=None):
    """int8 [128] key normalization shifts of one unit (after every unit's
    fp16 slots in the same buffer)."""
    h = _host(cache, layer, host)
    off = h.units * 2 * (scap + wcap) * 128 * 2 + u * 128
    return h.fp16[off:off + 128].view(np.int8)


def record_tail_is_zero(body_unit, lay, nb, k_inner, k_group, v_group, outk, k_hi, kb):
    """The per-token sections of the slots past the last body token of the
    unit's last (partly filled) block are zero (include/kvq.h record layout)."""
    if nb % 32 == 0:
        return True
    R = lay["record_bytes"]
    r = body_unit[(nb // 32) * R:(nb // 32 + 1) * R]
    f = nb % 32
    parts = []
    if kb != 3:
        rb = lay["k_row_bytes"]
        parts.append(r[lay["k_codes"] + f * rb:lay["k_codes"] + 32 * rb])
    if k_inner:
        ng = 128 // k_group
        parts.append(r[lay["k_meta"] + f * ng * 4:lay["k_meta"] + 32 * ng * 4])
    vm = r[lay["v_meta"]:].view(np.uint16)[:2 * (128 // v_group) * 32].reshape(-1, 32)
    parts.append(vm[:, f:].view(np.uint8).ravel())
    if outk:
        for sec in ("k_out", "v_out"):
            parts.append(r[lay[sec] + f * outk * 4:lay[sec] + 32 * outk * 4])
    if k_hi:
        wpt = k_hi * k_group // 2
        parts.append(r[lay["k_ext"] + f * wpt:lay["k_ext"] + 32 * wpt])
        parts.append(r[lay["k_sel"] + f:lay["k_sel"] + 32])
    return all(not np.any(p) for p in parts)


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    den = np.max(np.abs(ref), axis=-1)
    return np.max(np.abs(got - ref), axis=-1) / np.where(den == 0, 1.0, den)


def check_unit(wl, cache, outs, layer, u, steps=None, check_steps=None, label="", host=None,
               check_tail=False):
    """Bit-exact codes/params/outliers/fp16 area and per-step outputs of one unit."""
    b, h = divmod(u, wl.Hkv)
    host = _host(cache, layer, host)
    ref = O.run_unit(wl, layer, b, h, steps=steps, only_steps=check_steps)
    enc, nb = ref["enc"], ref["nb_final"]
    body, lay = unit_body(cache, layer, u, host)
    kb, vb = wl.bit_pairs()[layer]
    k_hi = wl.k_hi_groups if (wl.k_mode == "inner" and kb == 4) else 0
    got = unpack_unit(body, lay, kb, vb, nb, wl.k_mode == "inner", wl.k_group, wl.v_group, wl.outliers,
                      k_hi)
    for key in ("kcodes", "kmeta", "vcodes", "vmeta") + (("kwidth",) if k_hi else ()):
        g, r = got[key], enc[key]
        assert g.shape == r.shape, (label, key, g.shape, r.shape)
        bad = np.argwhere(g != r)
        assert bad.size == 0, (label, key, "mismatches", bad.shape[0], bad[:5].tolist(),
                               g[tuple(bad[0])], r[tuple(bad[0])])
    if wl.outliers:
        for key in ("kocol", "koval", "vocol", "voval"):
            assert np.array_equal(got[key], enc[key]), (label, key)
    if check_tail:
        assert record_tail_is_zero(body, lay, nb, wl.k_mode == "inner", wl.k_group, wl.v_group,
                                   wl.outliers, k_hi, kb), (label, "stale bytes past the last token")
    # fp16 sinks + window ring hold the exact (rotated, for values) tokens
    n, s_eff, nbody, r = host.state
    assert (n, s_eff, nbody) == (ref["n_final"], ref["s_eff"], nb)
    scap, wcap = lay["sink_cap"], lay["window_cap"]
    if ref.get("kshift") is not None:
        assert np.array_equal(unit_kshift(cache, layer, u, scap, wcap, host), ref["kshift"]), (label, "kshift")
    fk, fv = unit_fp16(cache, layer, u, scap, wcap, host)
    for p in list(range(s_eff)) + list(range(s_eff + nb, n)):
        slot = p if p < s_eff else scap + (p - s_eff) % wcap
        assert np.array_equal(fk[slot], ref["K"][p]), (label, "fp16 K", p)
        assert np.array_equal(fv[slot], enc["vrot"][p]), (label, "fp16 V", p)
    worst = 0.0
    for i, o_ref in ref["out"].items():
        o = outs[layer][i]
        o = o[u] if isinstance(o, dict) else o[b, h * wl.gq:(h + 1) * wl.gq]
        e = rel_err(o.double().numpy(), o_ref)
        worst = max(worst, float(e.max()))
        assert e.max() <= TOL, (label, "step", i, e.max())
    return worst


def check_units(wl, cache, outs, layer, units, check_steps=None, label="", threads=16):
    """check_unit over many units on a thread pool (the oracle's ctypes calls
    and numpy release the GIL).  Returns (worst row error, unit)."""
    from concurrent.futures import ThreadPoolExecutor
    host = HostLayer(cache, layer)

    def one(u):
        return check_unit(wl, cache, outs, layer, u, check_steps=check_steps, label=f"{label} u{u}",
                          host=host), u

    with ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(one, units))
    return max(res)
