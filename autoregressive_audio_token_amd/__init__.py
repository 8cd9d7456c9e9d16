"""Decode-step hot path of a Parler-TTS-style multi-codebook audio-token decoder
on AMD Instinct MI355X (gfx950).

The compute lives in libdecstep.so (HIP kernels behind a C ABI, declared in
include/decstep.h); ``decstep`` is its thin ctypes binding.  The binding (and
with it the library) loads on first use of any of its names, so the ``build``
module can run before the library exists; that first use fails with an
ImportError if the library has not been built.
"""
import importlib


def __getattr__(name):
    if name.startswith("__"):
        raise AttributeError(name)
    if name == "build":
        # `from autoregressive_audio_token_amd import build` asks for this attribute first;
        # answering through the binding would load the old library before the compile,
        # and the process would keep that copy (a second load of the path returns it)
        return importlib.import_module(__name__ + ".build")
    mod = importlib.import_module(__name__ + ".decstep")
    if name == "decstep":
        return mod
    try:
        return getattr(mod, name)
    except AttributeError:
        raise AttributeError(f"module {__name__!r} has no attribute {name!r}") from None
