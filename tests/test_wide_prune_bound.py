"""The lower bound the wide sampler prunes with, checked on the CPU (the mathematics the
kernel relies on; the kernel itself is checked against the oracle on the GPU).

Keys are the sampler's order-preserving uint32 map of float32 values.  With the row laid
out as entry i in lane i % 64, for t = ceil(k / 64) and t + 1: a_l is lane l's t-th largest
key (0 when it holds fewer than t), c = ceil(k / t), and the bound is the c-th largest a_l
found by a two-bits-a-step search to 18 leading bits that keeps count(a >= tau) >= c.  The
claims: the larger bound never exceeds the k-th largest key, so at least k keys survive and
every entry the kept set can hold (ties at the k-th key included) survives.
"""
import numpy as np
import pytest


def _order_keys(x):
    b = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    return np.where((b >> 31) == 1, (~b) & 0xFFFFFFFF, b | 0x80000000)


def _search(vals, c, stop=14):
    tau = 0
    for bit in range(31, stop, -2):
        cand = [tau | (m << (bit - 1)) for m in (1, 2, 3)]
        counts = [int((vals >= x).sum()) for x in cand]
        for x, n in zip(cand[::-1], counts[::-1]):
            if n >= c:
                tau = x
                break
    return tau


def _bound(keys, k):
    V = len(keys)
    slots = -(-V // 64)
    lanes = np.zeros((slots, 64), np.uint64)
    lanes.reshape(-1)[:V] = keys
    srt = np.sort(lanes, axis=0)[::-1]           # per lane, descending
    t0 = -(-k // 64)
    b = [_search(srt[t - 1], -(-k // t)) for t in (t0, t0 + 1) if t <= slots]
    return max(max(b), 1)


@pytest.mark.parametrize("seed", range(6))
def test_bound_never_exceeds_the_kth_key(seed):
    rng = np.random.default_rng(seed)
    for trial in range(40):
        V = int(rng.choice([520, 1089, 3000, 4096]))
        x = rng.standard_normal(V).astype(np.float32) * float(rng.choice([0.5, 3.0, 20.0]))
        kind = trial % 4
        if kind == 1:
            x = np.round(x)                      # ties
        elif kind == 2:
            x[:] = 0.25                          # a flat row
        elif kind == 3:
            x = -np.abs(x)                       # negative values only
        keys = _order_keys(x)
        k = int(rng.integers(65, 257))
        thr = _bound(keys, k)
        kth = np.sort(keys)[::-1][k - 1]
        assert thr <= kth, (V, k, kind)
        assert int((keys >= thr).sum()) >= k


def test_the_key_map_preserves_order():
    x = np.array([-np.inf, -3.5, -1e-30, -0.0, 0.0, 1e-30, 2.0, np.inf], np.float32)
    keys = _order_keys(x)
    assert np.all(np.diff(keys.astype(np.int64)[[0, 1, 2, 3, 5, 6, 7]]) > 0)
