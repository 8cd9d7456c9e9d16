"""Pins for oracle/heads.py (merged LM head, merged embedding lookup), CPU only."""
import math

import numpy as np

from oracle import heads
from workloads import gen


def _bf16(x):
    return gen.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_lm_head_brute_force_fsum():
    rng = np.random.default_rng(1)
    B, n_cb, Vs, V, D = 2, 3, 8, 7, 16
    h = _bf16(rng.standard_normal((B, D)))
    W = _bf16(rng.standard_normal((n_cb, Vs, D)))
    got = heads.lm_head(h, W, V)
    hf = h.astype(np.uint32) << 16
    Wf = W.astype(np.uint32) << 16
    hv = hf.view(np.float32).astype(np.float64)
    Wv = Wf.view(np.float32).astype(np.float64)
    for b in range(B):
        for c in range(n_cb):
            for v in range(V):
                want = math.fsum(hv[b, d] * Wv[c, v, d] for d in range(D))
                assert abs(got[b, c, v] - want) <= 1e-12 * max(1.0, abs(want))
    assert got.shape == (B, n_cb, V)          # padding rows of W are not part of the result


def test_lm_head_closed_forms():
    D, V = 8, 5
    h = np.arange(1, D + 1, dtype=np.float32)[None]
    W = np.zeros((2, 6, D), np.float32)
    for v in range(V):
        W[0, v, v] = 1.0                      # one-hot rows pick entries of h
    W[1, :, :] = 1.0                          # all-ones rows give the sum of h
    W[0, 5, :] = 1e30                         # a padding row that must not matter
    got = heads.lm_head(h, W, V)
    assert got[0, 0].tolist() == [1, 2, 3, 4, 5]
    assert got[0, 1].tolist() == [36.0] * V
    # linearity in h
    rng = np.random.default_rng(2)
    W2 = rng.standard_normal((2, 6, D)).astype(np.float32)
    a, b = rng.standard_normal((1, D)).astype(np.float32), rng.standard_normal((1, D)).astype(np.float32)
    lhs = heads.lm_head(a + b, W2, V)
    rhs = heads.lm_head(a.astype(np.float64), W2, V) + heads.lm_head(b.astype(np.float64), W2, V)
    assert np.allclose(lhs, rhs, rtol=1e-6, atol=1e-6)


def test_embed_hand_built_and_out_of_range():
    n_cb, V, D = 3, 4, 2
    E = np.zeros((n_cb, V, D), np.float32)
    for c in range(n_cb):
        for v in range(V):
            E[c, v] = [100 * c + v, -(100 * c + v)]
    toks = np.array([[1, 2, 3], [0, -1, 4]])
    got = heads.embed(toks, E)
    assert got[0].tolist() == [1 + 102 + 203, -(1 + 102 + 203)]
    assert got[1].tolist() == [0.0, 0.0]      # token 0 of codebook 0 is row 0 (zeros); -1 and 4 skip
    got = heads.embed(np.array([[0, 0, 0]]), E)
    assert got[0].tolist() == [0 + 100 + 200, -(0 + 100 + 200)]


def test_embed_bf16_exact_decode():
    E = _bf16(np.array([[[1.5, -2.0]], [[0.25, 8.0]]], np.float32))   # [2, 1, 2]
    assert heads.embed(np.array([[0, 0]]), E)[0].tolist() == [1.75, 6.0]
