"""Seeded synthetic inputs for the packed-KV decode workloads.

This module is the one piece shared by the CPU oracle's tests and the GPU
path's tests and benchmark: it only draws numbers.  It holds none of the
quantization or attention arithmetic.

Generator: a counter-based SplitMix64 stream.  Element ``idx`` of a logical
tensor keyed by ``key`` is ``mix64(key + (idx + 1) * GOLDEN)``, where ``mix64``
is the SplitMix64 output function (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014).  Because every element is a
pure function of its coordinates, any slice can be regenerated on any device,
in any order, bit for bit.

Normal and Student-t(3) draws go through 65536-entry inverse-CDF tables of
fp16 values indexed by the top 16 bits of the hash.  A table lookup is exact
on every device, so the CPU and GPU copies of a slice are identical (an
in-kernel Box-Muller would depend on each device's ``log``/``cos``).
"""
from __future__ import annotations

import math
import statistics

import numpy as np
import torch

M64 = (1 << 64) - 1
GOLDEN_U = 0x9E3779B97F4A7C15
C1_U = 0xBF58476D1CE4E5B9
C2_U = 0x94D049BB133111EB
T_CAP_LOG2 = 20          # positions per (b, h) stream: 2^20 > longest context + decode steps


def _s64(x: int) -> int:
    """Two's-complement int64 value of a uint64 bit pattern."""
    x &= M64
    return x - (1 << 64) if x >= (1 << 63) else x


GOLDEN = _s64(GOLDEN_U)
C1 = _s64(C1_U)
C2 = _s64(C2_U)


def mix64_py(z: int) -> int:
    """SplitMix64 output function on a Python int (uint64 semantics)."""
    z &= M64
    z = ((z ^ (z >> 30)) * C1_U) & M64
    z = ((z ^ (z >> 27)) * C2_U) & M64
    return z ^ (z >> 31)


def stream_py(key: int, i: int) -> int:
    """Element ``i`` of the stream ``key`` as a uint64."""
    return mix64_py((key + (i + 1) * GOLDEN_U) & M64)


def derive_key(*parts: int) -> int:
    """Fold integers into one uint64 stream key."""
    k = 0x243F6A8885A308D3
    for p in parts:
        k = mix64_py((k ^ (p & M64)) + GOLDEN_U)
    return k


def uniform_py(key: int, i: int) -> float:
    """U[0,1) with 53 random bits."""
    return (stream_py(key, i) >> 11) * (1.0 / (1 << 53))


# ---------------------------------------------------------------- torch side
def _srl(z: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 holding uint64 bits."""
    return torch.bitwise_and(torch.bitwise_right_shift(z, k), (1 << (64 - k)) - 1)


def mix64_t(z: torch.Tensor) -> torch.Tensor:
    z = torch.bitwise_xor(z, _srl(z, 30)) * C1
    z = torch.bitwise_xor(z, _srl(z, 27)) * C2
    return torch.bitwise_xor(z, _srl(z, 31))


def stream_t(key: int, idx: torch.Tensor) -> torch.Tensor:
    """Vectorised ``stream_py``: int64 tensor of uint64 bit patterns."""
    return mix64_t((idx + 1) * GOLDEN + _s64(key))


def _normal_table() -> np.ndarray:
    nd = statistics.NormalDist()
    p = [(i + 0.5) / 65536.0 for i in range(65536)]
    return np.array([nd.inv_cdf(x) for x in p], dtype=np.float64).astype(np.float16)


def _t3_cdf(t: np.ndarray) -> np.ndarray:
    x = t / math.sqrt(3.0)
    return 0.5 + (x / (1.0 + x * x) + np.arctan(x)) / math.pi


def _t3_table() -> np.ndarray:
    p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    lo = np.full_like(p, -1.0e4)
    hi = np.full_like(p, 1.0e4)
    for _ in range(120):
        mid = 0.5 * (lo + hi)
        below = _t3_cdf(mid) < p
        lo = np.where(below, mid, lo)
        hi = np.where(below, hi, mid)
    return (0.5 * (lo + hi)).astype(np.float16)


_TABLES: dict = {}


def table(name: str, device) -> torch.Tensor:
    dev = torch.device(device)
    k = (name, str(dev))
    if k not in _TABLES:
        src = _TABLES.get((name, "np"))
        if src is None:
            src = _normal_table() if name == "normal" else _t3_table()
            _TABLES[(name, "np")] = src
        _TABLES[k] = torch.from_numpy(src.copy()).to(dev)
    return _TABLES[k]


def draw_fp16(key: int, idx: torch.Tensor, dist: str) -> torch.Tensor:
    """fp16 draws for integer coordinates ``idx`` (same device as idx)."""
    bits = stream_t(key, idx)
    return table(dist, idx.device)[_srl(bits, 48)]


def partial_shuffle(key: int, n: int, count: int) -> list[int]:
    """First ``count`` entries of a seeded Fisher-Yates shuffle of range(n)."""
    a = list(range(n))
    for i in range(count):
        j = i + stream_py(key, i) % (n - i)
        a[i], a[j] = a[j], a[i]
    return sorted(a[:count])
