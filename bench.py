"""Benchmark: fused dequant decode attention over the packed KV cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C3|C2|C4|C5|...]

A step is one pass of the hot path for every layer in the stack: append one
token (quantizing a flush block when due) and decode attention of one query
per head over the whole packed cache.  The default workload is the largest
one: the Llama-3-8B shaped GQA stack (32 layers, batch 16, 32 query / 8 KV
heads, d=128, 8192-token context, each layer's (key, value) bit pair drawn
by seed from {KV8, K8V4, KV4, K4V2, KV2}); its 32 layer caches (about 6.6 GB
of packed cache) also keep consecutive decodes reading HBM rather than the
256 MB Infinity Cache.

The JSON line reports effective KV GB/s (algorithmic bytes of the decodes,
whole-job over the timed steps, appends included in the wall time), decode
tokens/s per layer, the decode's roofline fraction (algorithmic bytes per
launch over the HIP-event-timed duration of the decode call: split kernel +
log-sum-exp merge), the prefill (quantize/pack) throughput, and the CPU
oracle timed on this host on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
EVENT_EVERY = 4   # launch durations are sampled on every 4th timed step (see main)
METRIC = "fused dequant decode-attn: effective KV GB/s (% HBM peak), tokens/s per layer"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--workload", default="C3",
                   help="C1..C5, or a scheme variant: C5n (key normalization), C5m (mixed 4/8-bit "
                        "key groups), P5 (Hadamard 2-bit values on C2's layer), P5t (ternary values)")
    p.add_argument("--layers", type=int, default=None, help="layer caches in the stack")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="oracle time on all host threads (plus a third of it on one thread)")
    p.add_argument("--copy-calib", type=int, default=0,
                   help="only run a plain device copy of this many bytes (counter calibration)")
    return p.parse_args()


def workload(name, layers):
    from synth import workloads as W
    wl = W.get(name)
    if name == "C2":
        wl = wl.with_(L=layers or 8, fixed_pairs=((4, 2),) * (layers or 8))
    elif layers:
        pairs = wl.bit_pairs()
        wl = wl.with_(L=layers, fixed_pairs=tuple(pairs[:layers]) if len(pairs) >= layers else ())
    return wl


def decode_bytes(wl, layer, n, s_eff, nb, r):
    """Algorithmic bytes one decode must move (codes, per-group fp16 params,
    sparse outliers, fp16 sinks/window, q in, out)."""
    kb, vb = wl.bit_pairs()[layer]
    D = wl.D
    per_unit = nb * D * (kb + vb) / 8
    if wl.k_mode == "channel":
        per_unit += (nb // 32) * D * 4 + (nb % 32 > 0) * D * 4
    else:
        per_unit += nb * (D // wl.k_group) * 4
    per_unit += nb * (D // wl.v_group) * 4
    if wl.k_mode == "inner" and kb == 4 and wl.k_hi_groups:
        per_unit += nb * (wl.k_hi_groups * wl.k_group // 2 + 1)   # low nibbles + group mask
    per_unit += nb * wl.outliers * 4 * 2
    per_unit += (s_eff + r) * D * 2 * 2
    total = per_unit * wl.units + wl.B * wl.Hq * D * (2 + 4)
    if wl.nuq:
        total += 32
    return total


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_attention_quantize_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.startswith("kvq_decode") or f.endswith(".h"):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_record(name):
    path = os.path.join(ROOT, "profiles", f"decode_{name.lower()}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    """Threads for the oracle: the host's CPUs available to this process,
    at most 16 (one GPU's share of the host on the machines this runs on)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(wl, seconds):
    """The oracle (as it stands) decoding sampled units of one step on this
    host: all threads, then one thread."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle as O

    layer = 0
    sc = O.scheme_for(wl, layer)
    F = wl.flush
    s_eff, nb, r = O.state_prefill(wl.T, wl.sinks, wl.window, F)
    n = wl.T
    cores = host_threads()
    units = list(range(min(wl.units, 2 * cores)))
    prepared = []
    for u in units:
        b, h = divmod(u, wl.Hkv)
        K, V = O.unit_inputs(wl, layer, b, h, n)
        enc = O.encode_unit(sc, K, V, n, s_eff, nb)
        q = wl.q(layer, 0, b0=b, b1=b + 1, h0=h * wl.gq, h1=(h + 1) * wl.gq).reshape(wl.gq, wl.D)
        prepared.append((K, enc, q.double().numpy()))

    def one(item):
        K, enc, q = item
        Kh, Vh = O.dequant_unit(sc, K, enc, n, s_eff, nb)
        return O.attention(q, Kh, Vh, unrotate=bool(wl.v_hadamard))

    per_unit_bytes = (decode_bytes(wl, layer, n, s_eff, nb, r) - wl.B * wl.Hq * wl.D * 6) / wl.units \
        + wl.gq * wl.D * 6

    def timed(threads, budget, items):
        done, t0 = 0, time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            while True:
                list(ex.map(one, items))
                done += len(items)
                if time.perf_counter() - t0 >= budget:
                    break
        dt = time.perf_counter() - t0
        return per_unit_bytes * done / dt / 1e9, done, dt

    gbs, done, dt = timed(cores, seconds, prepared)
    gbs1, done1, dt1 = timed(1, seconds / 3, prepared[:1])
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "one_core_value": round(gbs1, 4),
            "sample": f"{done} (batch, kv-head) unit decodes of step 0 of layer 0 of {wl.name} "
                      f"(dequantize {n} tokens in binary64 + attention), {cores} threads, {dt:.1f} s; "
                      f"one thread: {done1} unit decodes in {dt1:.1f} s"}


def prefill_bytes(wl, layer, T, s_eff, nb, r):
    """Bytes one prefill of T tokens must move: read fp16 K and V of the
    prompt, write the nb packed body tokens and the s_eff + r fp16 sink /
    window tokens."""
    kb, vb = wl.bit_pairs()[layer]
    D = wl.D
    body = nb * D * (kb + vb) / 8
    body += ((nb // 32) * D * 4) if wl.k_mode == "channel" else nb * (D // wl.k_group) * 4
    body += nb * (D // wl.v_group) * 4 + nb * wl.outliers * 4 * 2
    if wl.k_mode == "inner" and kb == 4 and wl.k_hi_groups:
        body += nb * (wl.k_hi_groups * wl.k_group // 2 + 1)
    return wl.units * (T * D * 2 * 2 + body + (s_eff + r) * D * 2 * 2)


def read_ceiling(torch, dev, nbytes, splits, reps=24):
    """kvq_stream_read over nbytes (the decode's bytes per launch) with the
    decode's split count, rotating over eight buffers (more than the 256 MB
    Infinity Cache holds) so that every launch reads HBM; HIP events around
    each launch on the current stream."""
    from decode_attention_quantize_amd import kvq as K
    nbytes = max(4096, int(nbytes) // 4096 * 4096)
    nbuf = 8
    bufs = [torch.empty(nbytes + 256, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    ptrs = [b.data_ptr() + (-b.data_ptr()) % 256 for b in bufs]
    sink = torch.zeros(splits, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for i in range(nbuf):
        K.kvq_stream_read(ptrs[i], nbytes, splits, sink.data_ptr(), stream.cuda_stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        K.kvq_stream_read(ptrs[i % nbuf], nbytes, splits, sink.data_ptr(), stream.cuda_stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in ev[1:]]
    del bufs
    return nbytes / (sum(ms) / len(ms) / 1e3) / 1e9, nbytes


def copy_calibration(nbytes):
    import torch
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}))


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}); the path has no multi-GPU "
              "component in this build", file=sys.stderr)
        sys.exit(2)
    if a.copy_calib:
        copy_calibration(a.copy_calib)
        return
    import torch
    from decode_attention_quantize_amd import build as kb
    if kb.is_stale():
        kb.build()
    from decode_attention_quantize_amd import KVQCache, config_from_workload

    wl = workload(a.workload, a.layers)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    total_steps = a.warmup + a.steps
    if wl.append:
        wl = wl.with_(steps=total_steps)
    cfg = config_from_workload(wl, max_tokens=wl.T + total_steps)
    cache = KVQCache(cfg, wl.bit_pairs(), wl.codebooks(), device=dev)
    B, Hkv, T, D = wl.B, wl.Hkv, wl.T, wl.D
    stream = torch.cuda.current_stream(dev)
    # prefill: the first layer's prompt is quantized twice (the first pass
    # loads the kernels), then every layer's prefill is timed with events
    pre_ms, pre_bytes = [], []
    for l in range(wl.L):
        k = wl.k(l, 0, B, 0, Hkv, 0, T, device=dev).contiguous()
        v = wl.v(l, 0, B, 0, Hkv, 0, T, device=dev).contiguous()
        if l == 0:
            cache.prefill(l, k, v)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        cache.prefill(l, k, v)
        e1.record(stream)
        torch.cuda.synchronize()
        pre_ms.append(e0.elapsed_time(e1))
        _, s_eff0, nb0, r0 = cache.state(l)
        pre_bytes.append(prefill_bytes(wl, l, T, s_eff0, nb0, r0))
        del k, v
    torch.cuda.synchronize()
    # per-step inputs, generated before timing
    steps_in = []
    for i in range(total_steps):
        row = []
        for l in range(wl.L):
            kt = wl.k(l, 0, B, 0, Hkv, T + i, T + i + 1, device=dev).reshape(B, Hkv, D).contiguous()
            vt = wl.v(l, 0, B, 0, Hkv, T + i, T + i + 1, device=dev).reshape(B, Hkv, D).contiguous()
            q = wl.q(l, i, device=dev).contiguous()
            row.append((kt, vt, q))
        steps_in.append(row)
    outs = [torch.empty(B, wl.Hq, D, dtype=torch.float32, device=dev) for _ in range(wl.L)]
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(wl.L)] for _ in range(a.steps)]
    # Launch durations come from HIP events around the calls of every
    # EVENT_EVERY-th timed step.  Each timed event pair costs the GPU a few
    # microseconds between launches; around every call of the 32-layer stack
    # they took 13% of the whole-job time.  With one layer, the first timed
    # step is not sampled (see below).
    first = 1 if wl.L > 1 else 0
    skip = 0 if wl.L > 1 or a.steps < 2 else 1
    sampled = [k for k in range(skip, a.steps) if (k - skip) % EVENT_EVERY == 0]
    sampled_set = set(sampled)

    # kvq_append_decode_attn carries the append inside the decode launch for
    # layers that decode on the matrix-core kernel (no 3-bit codes); other
    # layers take the two calls, and the events then bracket the decode call
    # alone
    fused = wl.append and not wl.nuq and all(3 not in p for p in wl.bit_pairs())

    def step(i, ev=None, nbytes=None):
        # layer by layer, as a model step runs: the layer's new token enters
        # its cache and the query attends over it, in one
        # kvq_append_decode_attn call (one decode launch and its merge unless
        # a flush block is due).  Once the first call runs the host stays
        # ahead of the GPU, so the events around calls 2..L time the launches
        # themselves.
        for l in range(wl.L):
            kt, vt, q = steps_in[i][l]
            if wl.append and not fused:
                cache.append(l, kt, vt)
            if ev is not None:
                ev[l][0].record(stream)
            if wl.append and fused:
                cache.append_decode(l, kt, vt, q, outs[l])   # kvq_append_decode_attn
            else:
                cache.decode(l, q, outs[l])
            if ev is not None:
                ev[l][1].record(stream)
            if nbytes is not None:
                n, s_eff, nb, r = cache.state(l)
                nbytes.append(decode_bytes(wl, l, n, s_eff, nb, r))

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    nbytes = []
    t0 = time.perf_counter()
    for k, i in enumerate(range(a.warmup, total_steps)):
        step(i, events[k] if k in sampled_set else None, nbytes)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    # launch durations: decodes 2..L of each step (the first follows the host's
    # append calls and can include idle time).  With one layer, every decode
    # but the first timed one: the timed loop starts from an idle GPU, so the
    # first step's start event is passed before the host has launched that
    # decode; from the second step on the host runs a step ahead.
    kern_ms = [e0.elapsed_time(e1) for k in sampled for (e0, e1) in events[k][first:]]
    kern_bytes = [nb for k in sampled for nb in nbytes[k * wl.L + first:(k + 1) * wl.L]]
    kern_layer = [l for k in sampled for l in range(first, wl.L)]
    assert all(torch.isfinite(o).all() for o in outs)
    assert cache.nonfinite_rows() == 0
    # per (key, value) bit pair: mean decode call time and its roofline fraction
    by_pair = {}
    for ms, nb_, l in zip(kern_ms, kern_bytes, kern_layer):
        kb_, vb_ = wl.bit_pairs()[l]
        key = f"K{kb_}V{vb_}"
        t_, b_, c_ = by_pair.get(key, (0.0, 0.0, 0))
        by_pair[key] = (t_ + ms, b_ + nb_, c_ + 1)
    pairs_line = {k: {"us": round(t_ / c_ * 1e3, 2), "mb": round(b_ / c_ / 1e6, 2),
                      "frac": round(b_ / (t_ / 1e3) / 1e9 / HBM_PEAK_GBS, 4), "launches": c_}
                  for k, (t_, b_, c_) in sorted(by_pair.items())}

    total_bytes = sum(nbytes)
    value = total_bytes / dt / 1e9
    avg_kernel_s = sum(kern_ms) / len(kern_ms) / 1e3
    bytes_per_launch = sum(kern_bytes) / len(kern_bytes)
    achieved = bytes_per_launch / avg_kernel_s / 1e9
    tokens_per_s_layer = a.steps * wl.L * B / dt
    traffic = traffic_record(a.workload)
    ceil_gbs, ceil_bytes = read_ceiling(torch, dev, bytes_per_launch, 3072)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(dt / a.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: B={B} Hq={wl.Hq} Hkv={Hkv} D={D} context={T}+steps, "
                        f"pairs={sorted(set(wl.bit_pairs()))}, sinks={wl.sinks}, window={wl.window}, "
                        f"stack of {wl.L} layer caches; step = per layer append + decode",
            "layers": wl.L,
            "batch": B,
            "context": T,
        },
        "arith": "fp16 matrix-core operands (codes, q and p*s as exact hi+lo pairs), fp32 accumulation "
                 "and softmax",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s_per_layer": round(tokens_per_s_layer, 1),
        "decode_call_us": round(avg_kernel_s * 1e6, 2),
        "decode_by_pair": pairs_line,
        "prefill": {"gbs": round(sum(pre_bytes) / (sum(pre_ms) / 1e3) / 1e9, 1),
                    "frac": round(sum(pre_bytes) / (sum(pre_ms) / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                    "ms_per_layer": round(sum(pre_ms) / len(pre_ms), 3),
                    "mb_per_layer": round(sum(pre_bytes) / len(pre_bytes) / 1e6, 1),
                    "what": "kvq_quantize_prefill of each layer's prompt: fp16 K/V read + packed cache "
                            "and fp16 sinks/window written, HIP events"},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": round(bytes_per_launch),
            "kernel": ("kvq_append_decode_attn call: split-context decode kernel (storing the appended "
                       "token) + log-sum-exp merge kernel; a flush step adds the block quantization "
                       "(HIP events around the calls of every 4th step, launch gaps included)") if fused else
                      ("kvq_decode_attn call: split-context decode kernel + log-sum-exp merge kernel "
                       "(HIP events around the calls of every 4th step, launch gap included)"),
            "timed_launches": len(kern_ms),
            "frac_of_read_ceiling": round(achieved / ceil_gbs, 4),
        },
        "read_ceiling": {"gbs": round(ceil_gbs, 1), "frac": round(ceil_gbs / HBM_PEAK_GBS, 4),
                         "bytes": ceil_bytes,
                         "what": "kvq_stream_read: the decode's access pattern (3072 wavefronts, each a contiguous "
                                 "run of 4 KiB chunks as 1 KiB wave loads into an LDS ring) with no arithmetic, "
                                 "over the decode's bytes per launch, 8 rotating buffers, HIP events"},
    }
    if not a.no_cpu:
        line["cpu_baseline"] = cpu_baseline(W_for_cpu(a.workload), a.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    cache.close()


def W_for_cpu(name):
    from synth import workloads as W
    return W.get(name)


if __name__ == "__main__":
    main()
