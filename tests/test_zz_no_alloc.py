"""kvq_decode_attn_static (the decode entry point that allocates nothing)
against kvq_decode_attn on the same caches: two calls in a row, the second
over a smaller input, through the C ABI.  The two entry points run the same
kernels with the same split plan, so their outputs agree bit for bit; the
bound of the parity tests is asserted as well."""
import numpy as np
import pytest
import torch

from gpu_harness import TOL, rel_err, say
from synth import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cache(wl, steps):
    from decode_attention_quantize_amd import KVQCache, config_from_workload
    dev = torch.device("cuda")
    cache = KVQCache(config_from_workload(wl, max_tokens=wl.T + steps), wl.bit_pairs(), wl.codebooks(),
                     device=dev)
    B, Hkv, T = wl.B, wl.Hkv, wl.T
    for l in range(wl.L):
        cache.prefill(l, wl.k(l, 0, B, 0, Hkv, 0, T, device=dev).contiguous(),
                      wl.v(l, 0, B, 0, Hkv, 0, T, device=dev).contiguous())
    for i in range(steps):
        for l in range(wl.L):
            cache.append(l, wl.k(l, 0, B, 0, Hkv, T + i, T + i + 1, device=dev).reshape(B, Hkv, wl.D).contiguous(),
                         wl.v(l, 0, B, 0, Hkv, T + i, T + i + 1, device=dev).reshape(B, Hkv, wl.D).contiguous())
    return cache


def _compare(name, wl, steps=2):
    cache = _cache(wl, steps)
    worst = 0.0
    for l in range(wl.L):
        q = wl.q(l, steps, device="cuda").contiguous()
        ref = cache.decode(l, q)
        got = torch.full_like(ref, float("nan"))
        cache.decode_static(l, q, got)
        torch.cuda.synchronize()
        a, b = got.double().cpu().numpy(), ref.double().cpu().numpy()
        e = rel_err(a.reshape(-1, wl.D), b.reshape(-1, wl.D))
        worst = max(worst, float(e.max()))
        assert e.max() <= TOL, (name, l, e.max())
        assert np.array_equal(a, b), (name, l, "static and workspace decodes differ")
    say(f"[no-alloc] {name}: static == workspace decode, worst row difference {worst:.3e}")
    assert cache.nonfinite_rows() == 0
    from decode_attention_quantize_amd import kvq as K
    assert K.kvq_decode_nonfinite_rows(cache.handle, None, cache._stream()) == 0
    cache.close()


@pytest.mark.parametrize("first,second", [
    # matrix-core GQA layer, then a smaller MHA layer (fewer units, tokens, splits)
    ("C5r", "C2r"),
    # 3-bit table kernel with outliers and pre-RoPE keys, then a smaller one
    ("C4r", "C4s"),
    # every pair of the per-layer table, then one small layer
    ("C3r", "C1"),
    # the LDS-staged kernel (arrival counters in the static array's tail), twice
    ("uniform-3bit", "uniform-3bit-small"),
])
def test_static_decode_matches_workspace_decode(first, second):
    cases = {
        "C5r": W.C5.with_(B=2, Hq=16, Hkv=2, T=500, steps=2),
        "C2r": W.C2.with_(Hq=4, Hkv=4, T=1024, steps=2),
        "C4r": W.C4.with_(Hq=2, Hkv=2, T=1024, steps=2),
        "C4s": W.C4.with_(Hq=1, Hkv=1, T=300, steps=2),
        "C3r": W.C3.with_(L=5, B=2, Hq=8, Hkv=2, T=512, steps=2, fixed_pairs=W.PAIR_SET),
        "C1": W.C1.with_(append=True, steps=2),
        "uniform-3bit": W.C2.with_(Hq=2, Hkv=2, T=300, steps=2, fixed_pairs=((3, 3),)),
        "uniform-3bit-small": W.C2.with_(Hq=1, Hkv=1, T=100, steps=2, fixed_pairs=((3, 3),)),
    }
    _compare(first, cases[first])
    _compare(second, cases[second])


def test_static_decode_rejects_beyond_its_array():
    """More units than the static array's counter tail holds: refused before
    any launch, with the capacity status."""
    from decode_attention_quantize_amd import KVQError
    wl = W.C1.with_(B=2048, Hq=8, Hkv=8, T=40, window=32)     # 16384 units
    cache = _cache(wl, 0)
    q = wl.q(0, 0, device="cuda").contiguous()
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    with pytest.raises(KVQError) as e:
        cache.decode_static(0, q, out)
    assert e.value.status == 2
    cache.decode(0, q, out)                                   # the workspace entry point still serves it
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    cache.close()
