"""Pins for oracle/cache.py (writing the current token's row), CPU only: hand-built
expected arrays for every case of the length rule."""
import numpy as np

from oracle import cache


def test_append_writes_row_len_minus_one_only():
    NL, B, H, L, hd = 2, 3, 2, 4, 3
    k = np.arange(NL * B * H * L * hd, dtype=np.float32).reshape(NL, B, H, L, hd)
    v = -k.copy()
    kn = np.full((NL, B, H, hd), 1000.0, np.float32) + np.arange(NL * B * H * hd).reshape(NL, B, H, hd)
    vn = -kn
    want_k, want_v = k.copy(), v.copy()
    lens = [1, 4, 0]            # row 0; row 3 (last slot); nothing
    for layer in range(NL):
        for h in range(H):
            want_k[layer, 0, h, 0] = kn[layer, 0, h]
            want_v[layer, 0, h, 0] = vn[layer, 0, h]
            want_k[layer, 1, h, 3] = kn[layer, 1, h]
            want_v[layer, 1, h, 3] = vn[layer, 1, h]
    gk, gv = cache.append(kn, vn, k.copy(), v.copy(), lens)
    assert np.array_equal(gk, want_k) and np.array_equal(gv, want_v)


def test_append_out_of_range_lengths_write_nothing():
    k = np.zeros((1, 2, 1, 3, 2), np.float32)
    v = np.zeros_like(k)
    kn = np.ones((1, 2, 1, 2), np.float32)
    gk, gv = cache.append(kn, kn, k.copy(), v.copy(), [-1, 4])
    assert not gk.any() and not gv.any()
