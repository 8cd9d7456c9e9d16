"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library is rebuilt with its host pass instrumented (each sanitizer flag follows
-Xarch_host, so the device code is built exactly as usual) into _build/, cached by a hash of
the sources and flags.  tests/test_abi_cpu.py then runs again in a child process that loads
the instrumented library with the sanitizer runtime preloaded: every host-side validation
path of every entry point, the workspace arithmetic, the tuning overrides, the binding's
checks and the host key map, with any sanitizer report fatal.  The exhaustive sweep of the
key map over all 2^32 bit patterns stays in the plain run (it takes a minute under the
sanitizers); the other key-map tests run here.
"""
import hashlib
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from autoregressive_audio_token_amd import build as B  # noqa: E402

SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-shared-libasan"]


def _clang():
    for cand in ("/opt/rocm/llvm/bin/clang", shutil.which("clang") or ""):
        if cand and os.path.exists(cand):
            return cand
    return None


def _runtime():
    clang = _clang()
    if clang is None:
        return None
    path = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _flags():
    flags = [f for f in B.compile_flags() if f != "-O3"]
    return flags + ["-O1", "-g"] + SAN_FLAGS


def _build():
    h = hashlib.sha256(" ".join(_flags()).encode())
    for src in sorted(B.SOURCES) + sorted(os.listdir(B.CSRC)):
        p = os.path.join(B.CSRC, src)
        if os.path.isfile(p):
            h.update(open(p, "rb").read())
    h.update(open(os.path.join(ROOT, "include", "decstep.h"), "rb").read())
    out_dir = os.path.join(ROOT, "_build", "sanitized")
    out = os.path.join(out_dir, f"libdecstep_san_{h.hexdigest()[:16]}.so")
    if not os.path.exists(out):
        os.makedirs(out_dir, exist_ok=True)
        for old in os.listdir(out_dir):
            os.remove(os.path.join(out_dir, old))
        cmd = [B.hipcc_path(), *_flags(), "-shared", "-o", out + ".tmp",
               *[os.path.join(B.CSRC, s) for s in B.SOURCES]]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-3000:]
        os.replace(out + ".tmp", out)
    return out


@pytest.mark.skipif(__import__("torch").cuda.is_available(),
                    reason="the host checks hand fake addresses to the library: CPU only")
def test_abi_host_code_under_address_and_undefined_behaviour_sanitizers():
    rt = _runtime()
    if rt is None:
        pytest.skip("no clang sanitizer runtime")
    try:
        B.hipcc_path()
    except RuntimeError:
        pytest.skip("no hipcc")
    lib = _build()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_init" in syms and "__ubsan_handle" in syms, "the library is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, DECSTEP_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                          "-k", "not all_float32_bit_patterns"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in tail, tail
