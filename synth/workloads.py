"""The five synthetic decode workloads (shapes, schemes, data recipes).

Each workload fixes shapes, the quantization scheme per layer and the data
distribution; tensors are regenerated on demand from counter-based streams,
so a test can rebuild the inputs of one (layer, batch, kv-head) unit on the
CPU while the GPU holds the whole tensor.

Data recipe (the pages run real models; these stand in for their KV tensors):
  * q, K, V ~ N(0,1) rounded to fp16.
  * key outlier channels: a seeded set of channels per (layer, kv head), fixed
    across tokens, because key outliers are channel-aligned (KVTuner review,
    observation 2; KVQuant abstract).  They are either scaled (x8 / x10) or,
    for the long-context workload, drawn from Student-t(3).
  * decode-step tokens continue the same streams at positions T, T+1, ...
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch

from . import T_CAP_LOG2, derive_key, draw_fp16, partial_shuffle, stream_py, uniform_py

TID_K, TID_V, TID_Q = 1, 2, 3
TID_K_T3, TID_V_T3 = 101, 102
TID_CHANNELS, TID_PAIRS, TID_CODEBOOK = 10, 11, 12

# candidate per-layer (k_bits, v_bits) pairs: KV8, K8V4, KV4, K4V2, KV2
PAIR_SET = ((8, 8), (8, 4), (4, 4), (4, 2), (2, 2))


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    L: int
    T: int                 # prefill length
    steps: int             # decode steps
    append: bool = True    # append one token before each decode step
    sinks: int = 0
    window: int = 0
    k_mode: str = "channel"      # "channel" (groups of k_group tokens) | "inner" (k_group channels)
    k_group: int = 32
    v_group: int = 32
    v_hadamard: bool = False
    v_ternary: bool = False      # values as ternary levels {-s, 0, s} (2-bit codes)
    k_hybrid: bool = False
    sym_ratio: float = 0.1
    k_norm: bool = False         # per-channel key normalization from the prefill (inner keys)
    k_hi_groups: int = 0         # inner 4-bit keys: groups per token kept at 8 bits (mixed 4/8)
    pre_rope: bool = False
    rope_base: float = 10000.0
    nuq: bool = False
    outliers: int = 0            # sparse fp16 outliers per token vector (K and V)
    fixed_pairs: tuple = ()      # per-layer (kb, vb); empty -> seeded draw from PAIR_SET
    k_out_count: int = 0         # outlier channels per (layer, kv head) in K
    k_out_mode: str = "scale"    # "scale" | "t3"
    k_out_factor: float = 10.0
    v_out_count: int = 0
    v_out_factor: float = 10.0
    q_scale: float = 1.0
    notes: str = ""

    # ------------------------------------------------------------ scheme
    @property
    def units(self) -> int:
        return self.B * self.Hkv

    @property
    def gq(self) -> int:
        return self.Hq // self.Hkv

    @property
    def flush(self) -> int:
        return self.k_group if self.k_mode == "channel" else 1

    def bit_pairs(self) -> list:
        if self.fixed_pairs:
            assert len(self.fixed_pairs) == self.L
            return list(self.fixed_pairs)
        key = derive_key(self.seed, TID_PAIRS)
        return [PAIR_SET[stream_py(key, l) % len(PAIR_SET)] for l in range(self.L)]

    def codebooks(self):
        """uint16 [L][2][8] fp16 bit patterns (K, V) or None.

        Eight sorted fp16 levels in [0, 1] with L0 = 0 and L7 = 1; the six
        interior levels are U(0,1) draws rounded to fp16, redrawn on ties.
        """
        if not self.nuq:
            return None
        out = np.zeros((self.L, 2, 8), dtype=np.uint16)
        for l in range(self.L):
            for t in range(2):
                key = derive_key(self.seed, TID_CODEBOOK, l, t)
                attempt = 0
                while True:
                    u = [uniform_py(key, attempt * 6 + i) for i in range(6)]
                    lv = np.array([0.0] + u + [1.0], dtype=np.float64).astype(np.float16)
                    lv = np.sort(lv)
                    if len(set(lv.tolist())) == 8:
                        break
                    attempt += 1
                out[l, t] = lv.view(np.uint16)
        return out

    def outlier_channels(self, tensor: int, layer: int, h: int) -> list:
        n = self.k_out_count if tensor == TID_K else self.v_out_count
        if n == 0:
            return []
        key = derive_key(self.seed, TID_CHANNELS, tensor, layer, h)
        return partial_shuffle(key, self.D, n)

    # ------------------------------------------------------------ tensors
    def kv(self, tensor: int, layer: int, b0: int, b1: int, h0: int, h1: int,
           t0: int, t1: int, device="cpu") -> torch.Tensor:
        """fp16 [b1-b0][h1-h0][t1-t0][D] slice of K (tensor=1) or V (tensor=2)."""
        dev = torch.device(device)
        D = self.D
        b = torch.arange(b0, b1, device=dev, dtype=torch.int64).view(-1, 1, 1, 1)
        h = torch.arange(h0, h1, device=dev, dtype=torch.int64).view(1, -1, 1, 1)
        t = torch.arange(t0, t1, device=dev, dtype=torch.int64).view(1, 1, -1, 1)
        c = torch.arange(D, device=dev, dtype=torch.int64).view(1, 1, 1, -1)
        idx = (((b * self.Hkv + h) << T_CAP_LOG2) + t) * D + c
        x = draw_fp16(derive_key(self.seed, tensor, layer), idx, "normal")
        count = self.k_out_count if tensor == TID_K else self.v_out_count
        if count:
            for hi in range(h0, h1):
                ch = self.outlier_channels(tensor, layer, hi)
                sel = torch.tensor(ch, device=dev, dtype=torch.int64)
                j = hi - h0
                if tensor == TID_K and self.k_out_mode == "t3":
                    tid = TID_K_T3
                    x[:, j][..., sel] = draw_fp16(derive_key(self.seed, tid, layer),
                                                  idx[:, j][..., sel], "t3")
                else:
                    f = self.k_out_factor if tensor == TID_K else self.v_out_factor
                    x[:, j][..., sel] = (x[:, j][..., sel].float() * f).half()
        return x

    def k(self, layer, b0, b1, h0, h1, t0, t1, device="cpu"):
        return self.kv(TID_K, layer, b0, b1, h0, h1, t0, t1, device)

    def v(self, layer, b0, b1, h0, h1, t0, t1, device="cpu"):
        return self.kv(TID_V, layer, b0, b1, h0, h1, t0, t1, device)

    def q(self, layer: int, step: int, device="cpu", b0=0, b1=None, h0=0, h1=None) -> torch.Tensor:
        """fp16 [b][hq][D] decode query of a step (already position-encoded)."""
        dev = torch.device(device)
        b1 = self.B if b1 is None else b1
        h1 = self.Hq if h1 is None else h1
        D = self.D
        b = torch.arange(b0, b1, device=dev, dtype=torch.int64).view(-1, 1, 1)
        h = torch.arange(h0, h1, device=dev, dtype=torch.int64).view(1, -1, 1)
        c = torch.arange(D, device=dev, dtype=torch.int64).view(1, 1, -1)
        idx = (((b * self.Hq + h) << T_CAP_LOG2) + step) * D + c
        x = draw_fp16(derive_key(self.seed, TID_Q, layer), idx, "normal")
        if self.q_scale != 1.0:
            x = (x.float() * self.q_scale).half()
        return x

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


C1 = Workload(
    name="C1-tiny-mha", seed=1, B=1, Hq=1, Hkv=1, D=128, L=1, T=512, steps=1, append=False,
    window=32, fixed_pairs=((4, 4),), k_out_count=4, k_out_factor=8.0,
    notes="K4 per-channel G32, V4 per-token G32, last 32 tokens fp16; prefill then one decode")

C2 = Workload(
    name="C2-llama7b-mha-k4v2", seed=2, B=1, Hq=32, Hkv=32, D=128, L=1, T=32768, steps=64,
    sinks=4, window=128, fixed_pairs=((4, 2),), k_out_count=1, k_out_factor=10.0,
    notes="K4 per-channel G32, V2 per-token G32, 4 sinks + 128 recent fp16; 64 x (append, decode)")

C3 = Workload(
    name="C3-llama3-8b-gqa-mixed", seed=3, B=16, Hq=32, Hkv=8, D=128, L=32, T=8192, steps=64,
    k_out_count=3, k_out_factor=10.0,
    notes="per-layer seeded pair from {KV8,K8V4,KV4,K4V2,KV2}; K per-channel G32, V per-token G32")

C4 = Workload(
    name="C4-kvquant-131k", seed=4, B=1, Hq=32, Hkv=32, D=128, L=1, T=131072, steps=32,
    fixed_pairs=((3, 3),), pre_rope=True, nuq=True, outliers=2, k_out_count=3, k_out_mode="t3",
    notes="pre-RoPE K, 3-bit NUQ K (per-channel G32) and V (per-token G32), top-2 sparse fp16 outliers")

C5 = Workload(
    name="C5-70b-gqa-innerq-hadamard", seed=5, B=64, Hq=64, Hkv=8, D=128, L=1, T=16384, steps=4,
    k_mode="inner", k_group=64, k_hybrid=True, v_hadamard=True, fixed_pairs=((4, 2),),
    k_out_count=1, v_out_count=1,
    notes="K 4-bit inner groups of 64 hybrid sym/asym; V Hadamard-rotated 2-bit per-token G32")

ALL = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5}

# Scheme variants on the same shapes, measured beside the workloads above:
# InnerQ's per-channel key normalization and its mixed 4/8-bit key groups on
# C5; the Hadamard 2-bit page's pairing (int4 keys per channel, rotated 2-bit
# values) and its ternary-value control on C2's layer.
VARIANTS = {
    "C5n": C5.with_(name="C5n-70b-gqa-innerq-keynorm", k_norm=True),
    "C5m": C5.with_(name="C5m-70b-gqa-innerq-mixed48", k_hi_groups=1),
    "P5": C2.with_(name="P5-llama7b-mha-k4-hadamard-v2", v_hadamard=True),
    "P5t": C2.with_(name="P5t-llama7b-mha-k4-ternary-v", v_ternary=True),
}


def get(name: str) -> Workload:
    """A workload or a scheme variant by its short name."""
    return ALL[name] if name in ALL else VARIANTS[name]
