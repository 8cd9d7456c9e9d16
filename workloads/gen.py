"""Seeded synthetic inputs for the decode-step workloads.

Both the oracle and the HIP path consume exactly these arrays.  Nothing here
computes any part of the method: it only draws random numbers and stores them
in the layouts the boundary uses.

Every draw comes from ``numpy.random.Generator(PCG64(SeedSequence(t)))`` with
``t = (SEED_ROOT, cfg_id, stream, layer, index, step)``.  Normals are drawn as
float32, scaled by the workload's standard deviation (a power of two, so the
product is exact) and rounded once to bfloat16 with round-to-nearest-even;
the bf16 tensors are stored as their uint16 bit patterns.

Layouts (row-major, contiguous):
  q      [n_layers, B, H, hd]
  K, V   [n_layers, B, H, cap, hd]   slots >= the sequence's valid length hold
                                     ``invalid`` (NaN by default)
  logits [B, n_codebooks, vocab_stride] float32; columns >= vocab_valid hold
                                     ``pad_value``
  u      [B, n_codebooks] float32 in [0, 1)
  T      [B] float32
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from .configs import (SEED_ROOT, STREAM_Q_SELF, STREAM_K_SELF, STREAM_V_SELF,
                      STREAM_Q_CROSS, STREAM_K_CROSS, STREAM_V_CROSS,
                      STREAM_LENGTHS, STREAM_LOGITS, STREAM_UNIFORMS,
                      STREAM_TEMPERATURE, STREAM_K_NEW, STREAM_V_NEW, STREAM_HIDDEN,
                      STREAM_LM_W, STREAM_EMBED, Workload)

BF16_NAN = np.uint16(0x7FC0)


def rng_for(cfg_id, stream, layer=0, index=0, step=0):
    ss = np.random.SeedSequence([SEED_ROOT, int(cfg_id), int(stream), int(layer),
                                 int(index), int(step)])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs must be finite (normals always are).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _normals(rng, shape, std, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _elem_dtype(dtype):
    return np.uint16 if dtype == "bf16" else np.float32


def lengths(w: Workload):
    """Valid self and cross lengths per sequence, int32 [B] each."""
    if w.self_len is not None:
        s = np.full(w.batch, w.self_len, dtype=np.int32)
    else:
        lo, hi = w.self_len_range
        s = rng_for(w.cfg_id, STREAM_LENGTHS, 0, 0).integers(
            lo, hi, size=w.batch, endpoint=True).astype(np.int32)
    if w.cross_len is not None:
        c = np.full(w.batch, w.cross_len, dtype=np.int32)
    else:
        lo, hi = w.cross_len_range
        c = rng_for(w.cfg_id, STREAM_LENGTHS, 0, 1).integers(
            lo, hi, size=w.batch, endpoint=True).astype(np.int32)
    return s, c


def queries(w: Workload, kind: str, step: int = 0):
    """q for every layer: [n_layers, B, H, hd] (uint16 bf16 bits or float32)."""
    stream = STREAM_Q_SELF if kind == "self" else STREAM_Q_CROSS
    out = np.empty((w.n_layers, w.batch, w.heads, w.head_dim), dtype=_elem_dtype(w.dtype))
    for layer in range(w.n_layers):
        out[layer] = _normals(rng_for(w.cfg_id, stream, layer, 0, step),
                              (w.batch, w.heads, w.head_dim), w.qkv_std, w.dtype)
    return out


def kv_rows(w: Workload, kind: str, which: str, layer: int, b: int, n: int):
    """The first ``n`` cache rows of sequence ``b`` in ``layer``: [H, n, hd]."""
    if kind == "self":
        stream = STREAM_K_SELF if which == "k" else STREAM_V_SELF
        std = w.qkv_std
    else:
        stream = STREAM_K_CROSS if which == "k" else STREAM_V_CROSS
        std = w.cross_kv_std
    return _normals(rng_for(w.cfg_id, stream, layer, b), (w.heads, n, w.head_dim),
                    std, w.dtype)


def fill_rows(w: Workload, kind: str):
    """Rows drawn per sequence: the longest valid length any step of the workload reads."""
    return w.self_cap if kind == "self" else w.cross_cap


def cache(w: Workload, kind: str, which: str, lens, invalid="nan", threads=None,
          out=None):
    """Full static cache [n_layers, B, H, cap, hd] with the valid prefix of each sequence
    filled from the seeded draw and every other slot set to ``invalid`` ("nan" or "zero").
    """
    cap = w.self_cap if kind == "self" else w.cross_cap
    shape = (w.n_layers, w.batch, w.heads, cap, w.head_dim)
    if out is None:
        out = np.empty(shape, dtype=_elem_dtype(w.dtype))
    if invalid == "nan":
        out[...] = BF16_NAN if w.dtype == "bf16" else np.float32(np.nan)
    else:
        out[...] = 0
    lens = [min(max(int(n), 0), cap) for n in lens]

    def one(job):
        layer, b = job
        if lens[b] > 0:
            out[layer, b, :, :lens[b], :] = kv_rows(w, kind, which, layer, b, lens[b])

    jobs = [(layer, b) for layer in range(w.n_layers) for b in range(w.batch)]
    nthreads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(one, jobs))
    return out


def new_rows(w: Workload, which: str, step: int = 0):
    """The current token's self-attention key ("k") or value ("v") row for every
    (layer, sequence, head) at a step: [n_layers, B, H, hd]."""
    stream = STREAM_K_NEW if which == "k" else STREAM_V_NEW
    return _normals(rng_for(w.cfg_id, stream, 0, 0, step),
                    (w.n_layers, w.batch, w.heads, w.head_dim), w.qkv_std, w.dtype)


def hidden(w: Workload, D: int, step: int = 0):
    """The decoder's last hidden state at the last position: [B, D] bf16 bits, N(0,1)."""
    return _normals(rng_for(w.cfg_id, STREAM_HIDDEN, 0, 0, step), (w.batch, D), 1.0, "bf16")


def lm_head_weights(w: Workload, D: int):
    """Merged LM head [n_codebooks, vocab_stride, D] bf16 bits, N(0,1)/sqrt(D) (so logits
    are O(1)); padding rows are drawn too (the head never reads them)."""
    return _normals(rng_for(w.cfg_id, STREAM_LM_W), (w.n_codebooks, w.vocab_stride, D),
                    1.0 / 32 if D == 1024 else float(D) ** -0.5, "bf16")


def embedding_table(w: Workload, D: int):
    """Merged embeddings [n_codebooks, vocab_stride, D] bf16 bits, N(0,1)/8 (rows for
    every valid token and the fill token)."""
    return _normals(rng_for(w.cfg_id, STREAM_EMBED), (w.n_codebooks, w.vocab_stride, D),
                    0.125, "bf16")


def logits(w: Workload, step: int = 0, pad_value=1e30):
    """[B, n_codebooks, vocab_stride] float32, logit_std * N(0,1) in the valid columns."""
    x = np.full((w.batch, w.n_codebooks, w.vocab_stride), np.float32(pad_value),
                dtype=np.float32)
    r = rng_for(w.cfg_id, STREAM_LOGITS, 0, 0, step)
    v = r.standard_normal((w.batch, w.n_codebooks, w.vocab_valid), dtype=np.float32)
    v *= np.float32(w.logit_std)
    x[:, :, :w.vocab_valid] = v
    return x


def uniforms(w: Workload, step: int = 0):
    """[B, n_codebooks] float32 uniforms in [0, 1), drawn directly as float32."""
    r = rng_for(w.cfg_id, STREAM_UNIFORMS, 0, 0, step)
    return r.random((w.batch, w.n_codebooks), dtype=np.float32)


def temperatures(w: Workload):
    """[B] float32 sampling temperatures."""
    if w.temperature is not None:
        return np.full(w.batch, w.temperature, dtype=np.float32)
    lo, hi = w.temperature_range
    r = rng_for(w.cfg_id, STREAM_TEMPERATURE)
    return (lo + (hi - lo) * r.random(w.batch)).astype(np.float32)
