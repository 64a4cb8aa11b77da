"""Generated-code checks of the decode kernels' block loops (CPU only).

The decode kernels stream each split's blocks through an LDS ring filled by
load-to-LDS copies and count the copies in flight with explicit vmcnt waits.
Two code-generation hazards undo that ring without changing any result, so
only the generated code shows them:

- a spilled value reloaded inside the block loop: the reload is a vector
  memory access, and its wait also waits for every ring copy issued before it;
- a full vmcnt(0) wait inside the steady-state block loop (from a compiler-
  visible LDS access while copies are pending, or from a reload).

This test compiles the two matrix-core/table decode sources for gfx950 to
assembly and checks, for every kernel instance, the loop that holds most of
its matrix-core instructions (the steady-state block loop).
"""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from decode_attention_quantize_amd import build as B

SOURCES = {
    "kvq_decode_fast.hip": r"decode_mfma_kernel",
    "kvq_decode_lut.hip": r"decode_lut_kernel",
}


def _assembly(name: str, out_dir: str) -> str:
    src = os.path.join(B.CSRC, name)
    out = os.path.join(out_dir, name + ".s")
    flags = [f for f in B.FLAGS if f != "-fPIC"] + B.EXTRA.get(name, [])
    r = subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", out],
                       capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(r.stderr[-3000:])
    with open(out) as f:
        return f.read()


def _block_loops(asm: str, pattern: str):
    """Yield (kernel, loop lines) for the loop with the most MFMAs of each kernel."""
    for m in re.finditer(r"^(_Z\w+):", asm, re.M):
        name = m.group(1)
        if not re.search(pattern, name):
            continue
        body = asm[m.end():asm.index(".Lfunc_end", m.end())].split("\n")
        best = None
        for i, line in enumerate(body):
            if "Loop Header" not in line or "=>" not in line:
                continue
            label = line.split(":")[0]
            ends = [k for k, x in enumerate(body)
                    if re.search(r"s_(c)?branch\w*\s+" + re.escape(label) + r"\s*$", x.split(";")[0])]
            if not ends:
                continue
            seg = body[i:max(ends) + 1]
            n_mfma = sum("v_mfma" in x for x in seg)
            if best is None or n_mfma > best[0]:
                best = (n_mfma, seg)
        if best is not None and best[0] > 0:
            yield name, best[1]


@pytest.fixture(scope="module")
def assembly():
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d, ThreadPoolExecutor(len(SOURCES)) as ex:
        texts = dict(zip(SOURCES, ex.map(lambda n: _assembly(n, d), SOURCES)))
    return texts


@pytest.mark.parametrize("source", sorted(SOURCES))
def test_block_loops_keep_the_ring_in_flight(assembly, source):
    loops = list(_block_loops(assembly[source], SOURCES[source]))
    assert loops, f"no kernel block loop found in {source}"
    bad = []
    for name, seg in loops:
        reloads = sum("scratch_load" in x for x in seg)
        drains = sum(re.search(r"s_waitcnt\s+vmcnt\(0\)", x) is not None for x in seg)
        if reloads or drains:
            bad.append(f"{name}: {reloads} spill reloads, {drains} vmcnt(0) waits")
    assert not bad, "\n".join(bad)
