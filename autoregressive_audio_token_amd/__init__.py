"""Decode-step hot path of a Parler-TTS-style multi-codebook audio-token decoder
on AMD Instinct MI355X (gfx950).

The compute lives in libdecstep.so (HIP kernels behind a C ABI, declared in
include/decstep.h); ``decstep`` is its thin ctypes binding.  Importing this
package loads the library and fails if it has not been built.
"""
from . import decstep  # noqa: F401
from .decstep import *  # noqa: F401,F403
