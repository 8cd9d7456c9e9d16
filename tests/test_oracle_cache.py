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


def test_gather_paged_hand_built():
    # 2 layers, 3 physical blocks of 2 rows, 1 head, hd 1; values name (layer, block, row)
    pool = np.zeros((2, 3, 1, 2, 1), np.float32)
    for layer in range(2):
        for blk in range(3):
            for r in range(2):
                pool[layer, blk, 0, r, 0] = 100 * layer + 10 * blk + r
    table = np.array([[2, 0, 1], [1, 1, 1]], np.int32)
    got = cache.gather_paged(pool, table, 2, 1, 0, 0, 5)[:, 0]
    assert got.tolist() == [120, 121, 100, 101, 110]     # blocks 2, 0, 1 of layer 1
    got = cache.gather_paged(pool, table, 2, 0, 1, 0, 3)[:, 0]
    assert got.tolist() == [10, 11, 10]                  # a table may repeat a block
    assert cache.gather_paged(pool, table, 2, 0, 0, 0, 0).shape == (0, 1)


def test_gather_paged_identity_table_is_the_static_layout():
    # with table[b, i] = b * nb + i the pool holds exactly the static cache's rows
    rng = np.random.default_rng(3)
    NL, B, H, bs, nb, hd = 2, 3, 2, 4, 5, 3
    static = rng.standard_normal((NL, B, H, nb * bs, hd)).astype(np.float32)
    pool = np.zeros((NL, B * nb, H, bs, hd), np.float32)
    for b in range(B):
        for i in range(nb):
            pool[:, b * nb + i] = static[:, b, :, i * bs:(i + 1) * bs]
    table = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    for layer in range(NL):
        for b in range(B):
            for h in range(H):
                for n in (0, 1, 4, 5, 17, 20):
                    assert np.array_equal(cache.gather_paged(pool, table, bs, layer, b, h, n),
                                          static[layer, b, h, :n])
