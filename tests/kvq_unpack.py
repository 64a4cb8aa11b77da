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


def _section(recs: np.ndarray, off: int, nbytes: int) -> np.ndarray:
    """[nblk][nbytes] contiguous bytes of one record section."""
    return np.ascontiguousarray(recs[:, off:off + nbytes])


def _rows(sec: np.ndarray, bits: int) -> np.ndarray:
    """Token-major code rows (2/4/8 bits): [nblk][32 * D*bits/8] -> [nblk][32][D]."""
    r = sec.reshape(sec.shape[0], BT, D * bits // 8)
    if bits == 8:
        return r.copy()
    return _pair_split_fields(r.view(np.uint32), bits)


def _chunk3_fields(sec: np.ndarray) -> np.ndarray:
    """3-bit lane chunks: [nblk][64 * 24 bytes] -> [nblk][64 lanes][64 elements],
    element E at bits 3E..3E+2 of the chunk (little-endian bit stream)."""
    b = sec.reshape(sec.shape[0], 64, 24)
    bits = np.unpackbits(b, axis=2, bitorder="little")          # [nblk][64][192]
    f = bits.reshape(sec.shape[0], 64, 64, 3).astype(np.uint8)
    return f[..., 0] | (f[..., 1] << 1) | (f[..., 2] << 2)


# (token, channel) of element e of lane chunk l, for the three chunk layouts
_L, _E = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
# 3-bit keys: chunk l holds channels l and l + 64; element 2t + e is token t of channel l + 64e
_K3_TOK, _K3_CH = _E // 2, _L + 64 * (_E % 2)
# values (all widths): chunk l = 16g + n, element 8t + i is token 8g + i of channel 16t + n
_V_TOK, _V_CH = 8 * (_L // 16) + _E % 8, 16 * (_E // 8) + _L % 16


def _scatter(el: np.ndarray, tok: np.ndarray, ch: np.ndarray) -> np.ndarray:
    out = np.zeros((el.shape[0], BT, D), np.uint8)
    out[:, tok, ch] = el
    return out


def _vchunks(sec: np.ndarray, bits: int) -> np.ndarray:
    """Lane-chunk value codes [nblk][64 * 8*bits bytes] -> [nblk][32 tokens][D]."""
    nblk = sec.shape[0]
    if bits == 8:
        elems = sec.reshape(nblk, 64, 64)
    else:
        elems = _pair_split_fields(sec.view(np.uint32).reshape(nblk, 64, 2 * bits), bits)
    return _scatter(elems, _V_TOK, _V_CH)


def _mixed_keys(recs: np.ndarray, lay: dict, codes: np.ndarray, k_group: int, k_hi: int):
    """Mixed 4/8-bit key groups: the 8-bit groups named by each token's k_sel
    mask take (code plane field << 4) | low nibble from the token's k_ext
    slots (ascending group order).  Returns (codes, widths) [nblk][32][..]."""
    ng = D // k_group
    nblk = recs.shape[0]
    sel = _section(recs, lay["k_sel"], BT)
    wps = k_group // 8
    ext = _section(recs, lay["k_ext"], BT * k_hi * wps * 4).view(np.uint32).reshape(nblk, BT, k_hi, wps)
    lo = _pair_split_fields(ext, 4)                       # [nblk][32][k_hi][k_group]
    codes = codes.astype(np.uint8).copy()
    width = np.full((nblk, BT, ng), 4, np.uint8)
    for i in range(nblk):
        for t in range(BT):
            groups = [g for g in range(ng) if (sel[i, t] >> g) & 1]
            for slot, g in enumerate(groups[:k_hi]):
                cs = slice(g * k_group, (g + 1) * k_group)
                codes[i, t, cs] = (codes[i, t, cs] << 4) | lo[i, t, slot]
                width[i, t, g] = 8
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
    ngv = D // v_group
    flat = lambda a: a.reshape((nblk * BT,) + a.shape[2:])[:nb]
    out = {}
    kbytes = BT * D * kb // 8
    if kb == 3:
        kc = _scatter(_chunk3_fields(_section(recs, lay["k_codes"], 64 * 24)), _K3_TOK, _K3_CH)
    else:
        kc = _rows(_section(recs, lay["k_codes"], kbytes), kb)
    if k_hi:
        kc, kw = _mixed_keys(recs, lay, kc, k_group, k_hi)
        out["kwidth"] = flat(kw)
    out["kcodes"] = flat(kc)
    if vb == 3:
        vc = _scatter(_chunk3_fields(_section(recs, lay["v_codes"], 64 * 24)), _V_TOK, _V_CH)
    else:
        vc = _vchunks(_section(recs, lay["v_codes"], BT * D * vb // 8), vb)
    out["vcodes"] = flat(vc)
    if k_inner:
        ng = D // k_group
        out["kmeta"] = flat(_section(recs, lay["k_meta"], BT * ng * 4).view(np.uint16).reshape(nblk, BT, ng, 2))
    else:
        m16 = _section(recs, lay["k_meta"], 2 * D * 2).view(np.uint16).reshape(nblk, 2, D)
        out["kmeta"] = np.stack([m16[:, 0], m16[:, 1]], axis=-1)       # [nblk][D][2]
    v16 = _section(recs, lay["v_meta"], 2 * ngv * BT * 2).view(np.uint16).reshape(nblk, 2, ngv, BT)
    out["vmeta"] = flat(np.stack([v16[:, 0].transpose(0, 2, 1), v16[:, 1].transpose(0, 2, 1)], axis=-1))
    if outk:
        for key, name in (("k", "k_out"), ("v", "v_out")):
            w = _section(recs, lay[name], BT * outk * 4).view(np.uint32).reshape(nblk, BT, outk)
            out[key + "ocol"] = flat((w & 0xFFFF).astype(np.int32))
            out[key + "oval"] = flat((w >> 16).astype(np.uint16))
    return out
