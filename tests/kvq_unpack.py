"""Turn raw libkvq body records back into logical codes and parameters.

Written from the byte-layout specification in include/kvq.h (pair-split
words, lane chunks, 3-bit lane fields, SoA value parameters); it shares no code with
the kernels.  Used by the parity tests to compare packed GPU buffers with the
oracle's logical arrays bit for bit.
"""
from __future__ import annotations

import numpy as np

D = 128
BT = 32


def _pair_split_fields(words: np.ndarray, bits: int) -> np.ndarray:
    """[..., nwords] uint32 -> [..., nwords * 32/bits] fields in element order."""
    n = 32 // bits
    mask = (1 << bits) - 1
    out = np.empty(words.shape + (n,), dtype=np.uint8)
    for e in range(n):
        pos = (16 if e & 1 else 0) + bits * (e >> 1)
        out[..., e] = (words >> pos) & mask
    return out.reshape(words.shape[:-1] + (words.shape[-1] * n,))


def _rows(raw: np.ndarray, bits: int, nrows: int) -> np.ndarray:
    """Token-major code rows (2/4/8 bits): raw bytes [nrows * D*bits/8] -> [nrows][D]."""
    rb = D * bits // 8
    r = raw[: nrows * rb].reshape(nrows, rb)
    if bits == 8:
        return r.copy()
    return _pair_split_fields(r.view(np.uint32), bits)


def _chunk3_fields(raw: np.ndarray) -> np.ndarray:
    """3-bit lane chunks: 64 chunks of 24 bytes -> [64 lanes][64 elements],
    element E at bits 3E..3E+2 of the chunk (little-endian bit stream)."""
    b = raw[: 64 * 24].reshape(64, 24)
    bits = np.unpackbits(b, axis=1, bitorder="little")          # [64][192]
    f = bits.reshape(64, 64, 3).astype(np.uint8)
    return f[..., 0] | (f[..., 1] << 1) | (f[..., 2] << 2)


def _kchunks3(raw: np.ndarray) -> np.ndarray:
    """3-bit keys -> [32 tokens][D].  Chunk l holds channels l and l + 64;
    element 2*t + e is token t of channel l + 64*e."""
    el = _chunk3_fields(raw)
    out = np.zeros((BT, D), np.uint8)
    for lane in range(64):
        for e in range(64):
            out[e // 2, lane + 64 * (e % 2)] = el[lane, e]
    return out


def _vchunks3(raw: np.ndarray) -> np.ndarray:
    """3-bit values -> [32 tokens][D].  Chunk l = 16*g + n, element 8*t + i is
    token 8g + i of channel 16t + n."""
    el = _chunk3_fields(raw)
    out = np.zeros((BT, D), np.uint8)
    for lane in range(64):
        n, g = lane % 16, lane // 16
        for e in range(64):
            out[8 * g + e % 8, 16 * (e // 8) + n] = el[lane, e]
    return out


def _vchunks(raw: np.ndarray, bits: int) -> np.ndarray:
    """Lane-chunk value codes of one block -> [32 tokens][D]."""
    nbytes = 64 * 8 * bits
    words = raw[:nbytes].view(np.uint32).reshape(64, 2 * bits)
    if bits == 8:
        elems = raw[:nbytes].reshape(64, 64)
    else:
        elems = _pair_split_fields(words, bits)          # [64 lanes][64 elements]
    out = np.zeros((BT, D), np.uint8)
    for lane in range(64):
        for idx in range(64):
            j = 8 * (lane // 16) + (idx % 8)
            c = 16 * (idx // 8) + (lane % 16)
            out[j, c] = elems[lane, idx]
    return out


def _mixed_keys(r: np.ndarray, lay: dict, codes: np.ndarray, k_group: int, k_hi: int):
    """Mixed 4/8-bit key groups of one block: the 8-bit groups named by each
    token's k_sel mask take (code plane field << 4) | low nibble from the
    token's k_ext slots (ascending group order).  Returns (codes, widths)."""
    ng = D // k_group
    sel = r[lay["k_sel"]: lay["k_sel"] + BT]
    wps = k_group // 8
    ext = r[lay["k_ext"]: lay["k_ext"] + BT * k_hi * wps * 4].view(np.uint32).reshape(BT, k_hi, wps)
    lo = _pair_split_fields(ext, 4)                       # [32][k_hi][k_group]
    codes = codes.astype(np.uint8).copy()
    width = np.full((BT, ng), 4, np.uint8)
    for t in range(BT):
        groups = [g for g in range(ng) if (sel[t] >> g) & 1]
        for slot, g in enumerate(groups[:k_hi]):
            cs = slice(g * k_group, (g + 1) * k_group)
            codes[t, cs] = (codes[t, cs] << 4) | lo[t, slot]
            width[t, g] = 8
    return codes, width


def unpack_unit(body_unit: np.ndarray, lay: dict, kb: int, vb: int, nb: int, k_inner: bool,
                k_group: int, v_group: int, outk: int, k_hi: int = 0) -> dict:
    """Logical arrays of the first nb body tokens of one unit.

    body_unit: uint8 [nblk_cap * record_bytes] for that unit.
    Returns kcodes [nb][D], kmeta (per-channel [nb/32][D][2] or inner [nb][D/kg][2]),
    vcodes [nb][D], vmeta [nb][D/vg][2], kocol/koval/vocol/voval [nb][outk], and
    with mixed 4/8-bit key groups (k_hi > 0) kwidth [nb][D/kg].
    """
    R = lay["record_bytes"]
    nblk = (nb + BT - 1) // BT
    recs = body_unit[: nblk * R].reshape(nblk, R)
    kc, vc, km, vm, kw = [], [], [], [], []
    ko_c, ko_v, vo_c, vo_v = [], [], [], []
    ngv = D // v_group
    for i in range(nblk):
        r = recs[i]
        cnt = min(BT, nb - BT * i)
        if kb == 3:
            kc.append(_kchunks3(r[lay["k_codes"]:])[:cnt])
        elif k_hi:
            codes, width = _mixed_keys(r, lay, _rows(r[lay["k_codes"]:], kb, BT), k_group, k_hi)
            kc.append(codes[:cnt])
            kw.append(width[:cnt])
        else:
            kc.append(_rows(r[lay["k_codes"]:], kb, BT)[:cnt])
        if vb == 3:
            vc.append(_vchunks3(r[lay["v_codes"]:])[:cnt])
        else:
            vc.append(_vchunks(r[lay["v_codes"]:], vb)[:cnt])
        m16 = r[lay["k_meta"]:].view(np.uint16)
        if k_inner:
            ng = D // k_group
            km.append(m16[: BT * ng * 2].reshape(BT, ng, 2)[:cnt])
        else:
            km.append(np.stack([m16[:D], m16[D:2 * D]], axis=-1)[None])
        v16 = r[lay["v_meta"]:].view(np.uint16)
        s = v16[: ngv * BT].reshape(ngv, BT)
        z = v16[ngv * BT: 2 * ngv * BT].reshape(ngv, BT)
        vm.append(np.stack([s.T, z.T], axis=-1)[:cnt])
        if outk:
            k32 = r[lay["k_out"]:].view(np.uint32)[: BT * outk].reshape(BT, outk)[:cnt]
            v32 = r[lay["v_out"]:].view(np.uint32)[: BT * outk].reshape(BT, outk)[:cnt]
            ko_c.append((k32 & 0xFFFF).astype(np.int32))
            ko_v.append((k32 >> 16).astype(np.uint16))
            vo_c.append((v32 & 0xFFFF).astype(np.int32))
            vo_v.append((v32 >> 16).astype(np.uint16))
    cat = lambda xs, shape, dt: np.concatenate(xs) if xs else np.zeros(shape, dt)
    out = dict(
        kcodes=cat(kc, (0, D), np.uint8), vcodes=cat(vc, (0, D), np.uint8),
        kmeta=cat(km, (0, D, 2), np.uint16), vmeta=cat(vm, (0, ngv, 2), np.uint16),
    )
    if k_hi:
        out["kwidth"] = cat(kw, (0, D // k_group), np.uint8)
    if outk:
        out.update(kocol=cat(ko_c, (0, outk), np.int32), koval=cat(ko_v, (0, outk), np.uint16),
                   vocol=cat(vo_c, (0, outk), np.int32), voval=cat(vo_v, (0, outk), np.uint16))
    return out
