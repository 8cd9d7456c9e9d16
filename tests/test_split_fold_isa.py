"""The split-mode fold's ordering, held against the code the compiler emits (CPU only).

A chunk's workgroup publishes its partial state with agent-scope relaxed atomic stores,
waits for every one of them (s_waitcnt vmcnt(0)), and only then takes the sequence's ticket
with an agent-scope atomic add; the workgroup that draws the last ticket reads the states
with agent-scope relaxed atomic loads.  Under the AMDGPU memory model for GFX942/GFX950
(LLVM's AMDGPUUsage), agent-scope atomic loads and stores carry sc1 (device scope: written
through, and read past, the XCD's own L2), and an agent-scope release/acquire pair lowers to
an L2 write-back + s_waitcnt vmcnt(0) / an L2 invalidate.  The write-back and invalidate
serve only non-atomic data cached in an L2; with every shared access an sc1 atomic, what
remains is the wait, which the kernel has.  This test compiles the kernel and checks those
facts in its ISA, so a toolchain that lowers these atomics differently fails here instead of
silently.
"""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from autoregressive_audio_token_amd import build as B  # noqa: E402

VMEM = re.compile(r"^\s*(global|buffer|flat)_(load|store|atomic)")


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("isa") / "attn.s")
    flags = [f for f in B.compile_flags() if f != "-fPIC"]
    res = subprocess.run([B.hipcc_path(), *flags, "--cuda-device-only", "-S", "-o", out,
                          os.path.join(B.CSRC, "attn_decode.hip")], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    text = open(out).read().splitlines()
    bodies, name, cur = {}, None, []
    for ln in text:
        m = re.match(r"^(_ZN3dec18attn_decode_kernel\w+):", ln)
        if m:
            name, cur = m.group(1), []
            continue
        if name is not None:
            cur.append(ln)
            if "s_endpgm" in ln:
                bodies[name] = cur
                name = None
    assert len(bodies) >= 10, sorted(bodies)
    return bodies


def test_every_instantiation_publishes_waits_then_takes_the_ticket(kernels):
    for name, body in kernels.items():
        atomics = [i for i, ln in enumerate(body) if re.match(r"^\s*global_atomic_add\b", ln)]
        assert len(atomics) == 1, (name, len(atomics))
        a = atomics[0]
        # the nearest preceding full wait, with no vector memory access between it and the add
        waits = [i for i in range(a) if re.match(r"^\s*s_waitcnt\b.*vmcnt\(0\)", body[i])]
        assert waits, name
        assert not any(VMEM.match(body[i]) for i in range(waits[-1] + 1, a)), name
        # agent-scope relaxed stores (chunk states, ticket reset) and loads (chunk states)
        sc1_stores = [ln for ln in body if re.match(r"^\s*global_store_dword\w*\b.*\bsc1\b", ln)]
        sc1_loads = [ln for ln in body[a:] if re.match(r"^\s*global_load_dword\w*\b.*\bsc1\b", ln)]
        assert len(sc1_stores) >= 3, (name, sc1_stores)
        assert len(sc1_loads) >= 3, (name, sc1_loads)
        assert any(i > a for i, ln in enumerate(body)
                   if re.match(r"^\s*global_store_dword\w*\b.*\bsc1\b", ln)), name  # ticket reset
