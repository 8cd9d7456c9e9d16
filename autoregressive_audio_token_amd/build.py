"""Build libdecstep.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m autoregressive_audio_token_amd.build [--out PATH] [-D NAME=VALUE ...]
"""
import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdecstep.so")
SOURCES = ["attn_decode.hip", "sample_topk.hip", "heads.hip", "probe.hip", "decstep_abi.hip"]
ARCH = "gfx950"


def hipcc_path():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags(defines=()):
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             # no packed fp32 instructions in any generated code
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # floating point exactly as written: fused multiply-adds only where fmaf says so
             "-ffp-contract=off",
             "-Wall", "-Wno-unused-function", "-Werror=uninitialized",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    flags += [f"-D{d}" for d in defines]
    return flags


def build(out=LIB, defines=(), verbose=False):
    """Compile every source into one shared library; returns its path."""
    hipcc = hipcc_path()
    tmp = out + ".tmp"
    cmd = [hipcc, *compile_flags(defines), "-shared", "-o", tmp,
           *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.out, a.defines, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
