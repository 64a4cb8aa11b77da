"""Turn raw libkvq body records back into logical codes and parameters.

Written from the byte-layout specification in include/kvq.h (pair-split
words, lane chunks, bit planes, SoA value parameters); it shares no code with
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
    """Token-major code rows: raw bytes [nrows * D*bits/8] -> [nrows][D]."""
    rb = D * bits // 8
    r = raw[: nrows * rb].reshape(nrows, rb)
    if bits == 8:
        return r.copy()
    words = r.view(np.uint32)
    if bits == 3:
        planes = words.reshape(nrows, D // 32, 3)
        out = np.zeros((nrows, D // 32, 32), np.uint8)
        for p in range(3):
            bitsv = (planes[:, :, p:p + 1] >> np.arange(32, dtype=np.uint32)) & 1
            out |= (bitsv << p).astype(np.uint8)
        return out.reshape(nrows, D)
    return _pair_split_fields(words, bits)


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


def unpack_unit(body_unit: np.ndarray, lay: dict, kb: int, vb: int, nb: int, k_inner: bool,
                k_group: int, v_group: int, outk: int) -> dict:
    """Logical arrays of the first nb body tokens of one unit.

    body_unit: uint8 [nblk_cap * record_bytes] for that unit.
    Returns kcodes [nb][D], kmeta (per-channel [nb/32][D][2] or inner [nb][D/kg][2]),
    vcodes [nb][D], vmeta [nb][D/vg][2], kocol/koval/vocol/voval [nb][outk].
    """
    R = lay["record_bytes"]
    nblk = (nb + BT - 1) // BT
    recs = body_unit[: nblk * R].reshape(nblk, R)
    kc, vc, km, vm = [], [], [], []
    ko_c, ko_v, vo_c, vo_v = [], [], [], []
    ngv = D // v_group
    for i in range(nblk):
        r = recs[i]
        cnt = min(BT, nb - BT * i)
        kc.append(_rows(r[lay["k_codes"]:], kb, BT)[:cnt])
        if vb == 3:
            vc.append(_rows(r[lay["v_codes"]:], 3, BT)[:cnt])
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
    if outk:
        out.update(kocol=cat(ko_c, (0, outk), np.int32), koval=cat(ko_v, (0, outk), np.uint16),
                   vocol=cat(vo_c, (0, outk), np.int32), voval=cat(vo_v, (0, outk), np.uint16))
    return out
