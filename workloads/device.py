"""Stage the seeded workload arrays into device memory (torch tensors).

Plumbing only: copies, views and fills; no arithmetic of the method.  bf16
arrays travel as their uint16 bit patterns and are viewed as torch.bfloat16.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np
import torch

from . import gen
from .configs import Workload


def to_device(a, device, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a).to(device)
    return t if dtype is None else t.to(dtype)


def empty_cache(w: Workload, kind, device, fill=float("nan")):
    cap = w.self_cap if kind == "self" else w.cross_cap
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return torch.full((w.n_layers, w.batch, w.heads, cap, w.head_dim), fill, dtype=dt,
                      device=device)


def fill_cache(w: Workload, kind, which, lens, dst, threads=16):
    """Write the seeded valid prefix of every (layer, b) into a device cache ``dst``
    (slots past the valid prefix keep whatever ``dst`` holds)."""
    jobs = [(layer, b, int(lens[b])) for layer in range(w.n_layers) for b in range(w.batch)
            if int(lens[b]) > 0]

    def draw(job):
        layer, b, n = job
        return job, gen.kv_rows(w, kind, which, layer, b, n)

    with ThreadPoolExecutor(min(threads, os.cpu_count() or 1)) as ex:
        for (layer, b, n), rows in ex.map(draw, jobs):
            dst[layer, b, :, :n, :] = to_device(rows, dst.device)
    return dst


def step_inputs(w: Workload, device, self_lens=None, cross_lens=None, invalid=float("nan"),
                step=0, fill_lens=None):
    """Every device tensor one decode step needs.

    ``fill_lens`` (self, cross) chooses how many rows per sequence are drawn into the
    caches (default: the valid lengths); ``self_lens``/``cross_lens`` default to the
    workload's.
    """
    s_len, c_len = gen.lengths(w)
    if self_lens is not None:
        s_len = np.asarray(self_lens, dtype=np.int32)
    if cross_lens is not None:
        c_len = np.asarray(cross_lens, dtype=np.int32)
    fs, fc = fill_lens if fill_lens is not None else (s_len, c_len)
    fs = np.minimum(np.maximum(np.asarray(fs), 0), w.self_cap)
    fc = np.minimum(np.maximum(np.asarray(fc), 0), w.cross_cap)
    d = dict(self_len_host=s_len, cross_len_host=c_len)
    d["q_self"] = to_device(gen.queries(w, "self"), device)
    d["q_cross"] = to_device(gen.queries(w, "cross"), device)
    for kind, lens in (("self", fs), ("cross", fc)):
        for which in ("k", "v"):
            d[f"{which}_{kind}"] = fill_cache(w, kind, which, lens,
                                              empty_cache(w, kind, device, invalid))
    d["len"] = torch.from_numpy(s_len.astype(np.int32)).to(device)
    d["enc_len"] = torch.from_numpy(c_len.astype(np.int32)).to(device)
    d["logits"] = to_device(gen.logits(w, step), device)
    d["uniforms"] = to_device(gen.uniforms(w, step), device)
    d["temperature"] = to_device(gen.temperatures(w), device)
    d["step"] = torch.full((w.batch,), step, dtype=torch.int32, device=device)
    return d
