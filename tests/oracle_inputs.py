"""Host-side inputs for the oracle, drawn straight from the seeded generators.

The oracle never sees a value that passed through the GPU: every row it needs is
regenerated here from ``workloads.gen`` (the same seeds the device tensors were
filled from).
"""
import numpy as np

from oracle import attn as oattn
from workloads import gen


def _f64(x, dtype):
    if dtype == "bf16":
        return oattn.bf16_bits_to_f64(x)
    return np.asarray(x, np.float32).astype(np.float64)


class RowSource:
    """Lazily regenerates per-(layer, b) cache blocks of a workload."""

    def __init__(self, w, fill_self, fill_cross, step=0):
        self.w = w
        self.fill = {"self": np.asarray(fill_self), "cross": np.asarray(fill_cross)}
        self.q = {k: gen.queries(w, k, step) for k in ("self", "cross")}
        self._kv = {}

    def kv(self, kind, which, layer, b):
        key = (kind, which, layer, b)
        if key not in self._kv:
            cap = self.w.self_cap if kind == "self" else self.w.cross_cap
            n = int(min(max(int(self.fill[kind][b]), 0), cap))
            self._kv[key] = gen.kv_rows(self.w, kind, which, layer, b, n)
        return self._kv[key]

    def expected(self, kind, lens, rows, scale=None):
        """Oracle outputs [len(rows), hd] (float64) for (layer, b, h) rows."""
        w = self.w
        scale = w.scale if scale is None else scale
        cap = w.self_cap if kind == "self" else w.cross_cap
        out = np.zeros((len(rows), w.head_dim))
        for r, (layer, b, h) in enumerate(rows):
            n = min(int(lens[b]), cap)
            if n <= 0:
                continue
            q = _f64(self.q[kind][layer, b, h], w.dtype)
            K = _f64(self.kv(kind, "k", layer, b)[h, :n], w.dtype)
            V = _f64(self.kv(kind, "v", layer, b)[h, :n], w.dtype)
            out[r] = oattn.attend_one(q, K, V, n, scale)
        return out


def all_rows(w):
    return [(layer, b, h) for layer in range(w.n_layers) for b in range(w.batch)
            for h in range(w.heads)]


def sampled_rows(w, count, seed=0):
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(w.batch):                 # every sequence at least once
        rows.add((int(rng.integers(w.n_layers)), b, int(rng.integers(w.heads))))
    while len(rows) < count:
        rows.add((int(rng.integers(w.n_layers)), int(rng.integers(w.batch)),
                  int(rng.integers(w.heads))))
    return sorted(rows)
