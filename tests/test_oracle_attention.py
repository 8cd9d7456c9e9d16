"""Pins for the attention oracle (CPU only).

Each test checks oracle.attention against something other than itself: exact
bfloat16 decodings, a library implementation of masked scaled-dot-product
attention, closed forms that follow from the definition, and invariants.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attn as A
from workloads import configs, gen


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


# -- bfloat16 decoding: exact values from the format's definition -------------

def test_bf16_decode_exact_values():
    bits = np.array([0x3F80, 0xC000, 0x3FC0, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x4049,
                     0x3E00], dtype=np.uint16)
    want = [1.0, -2.0, 1.5, math.inf, -math.inf, 2.0 ** -133, -0.0, 3.140625, 0.125]
    got = A.bf16_bits_to_f64(bits)
    for g, w in zip(got, want):
        assert g == w and math.copysign(1, g) == math.copysign(1, w)
    assert np.isnan(A.bf16_bits_to_f64(np.array([0x7FC0], np.uint16)))[0]


def test_bf16_rounding_of_generator_matches_torch():
    # The generator's rounding (input preparation) agrees with torch's bf16 cast.
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 3).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 65504.0]  # exact ties
    ours = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# -- library special case: torch SDPA in float64 with a boolean prefix mask ------

@pytest.mark.parametrize("seed", range(6))
def test_matches_torch_sdpa_float64(seed):
    rng = np.random.default_rng(seed)
    NL, B, H, cap, hd = 2, 3, 2, 40, int(rng.choice([1, 2, 8, 64]))
    q = _rand(rng, NL, B, H, hd).astype(np.float32)
    K = _rand(rng, NL, B, H, cap, hd).astype(np.float32)
    V = _rand(rng, NL, B, H, cap, hd).astype(np.float32)
    lens = rng.integers(1, cap + 1, size=B)
    scale = float(rng.uniform(0.05, 1.0))
    got = A.attention(q, K, V, lens, scale, "f32")

    tq = torch.from_numpy(q.astype(np.float64)).reshape(NL * B * H, 1, 1, hd)
    tk = torch.from_numpy(K.astype(np.float64)).reshape(NL * B * H, 1, cap, hd)
    tv = torch.from_numpy(V.astype(np.float64)).reshape(NL * B * H, 1, cap, hd)
    mask = torch.zeros(NL, B, H, 1, 1, cap, dtype=torch.bool)
    for b in range(B):
        mask[:, b, :, :, :, :lens[b]] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask.reshape(NL * B * H, 1, 1, cap), scale=scale)
    ref = ref.reshape(NL, B, H, hd).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


# -- closed forms -------------------------------------------------------------

def test_single_valid_key_returns_its_value():
    rng = np.random.default_rng(1)
    K = _rand(rng, 10, 64)
    V = _rand(rng, 10, 64)
    q = _rand(rng, 64)
    out = A.attend_one(q, K, V, 1, 0.125)
    assert np.array_equal(out, V[0])


def test_two_keys_is_a_sigmoid_blend():
    rng = np.random.default_rng(2)
    for _ in range(20):
        K = _rand(rng, 2, 64)
        V = _rand(rng, 2, 64)
        q = _rand(rng, 64)
        scale = 0.3
        s0, s1 = scale * float(K[0] @ q), scale * float(K[1] @ q)
        a0 = 1.0 / (1.0 + math.exp(s1 - s0))
        want = a0 * V[0] + (1 - a0) * V[1]
        assert np.allclose(A.attend_one(q, K, V, 2, scale), want, rtol=1e-13, atol=1e-14)


def test_equal_scores_give_the_mean_value():
    rng = np.random.default_rng(3)
    K = np.tile(_rand(rng, 1, 64), (50, 1))          # every key identical
    V = _rand(rng, 50, 64)
    q = _rand(rng, 64)
    for n in (1, 7, 50):
        assert np.allclose(A.attend_one(q, K, V, n, 0.125), V[:n].mean(axis=0),
                           rtol=1e-13, atol=1e-14)
    # scale 0 makes every score equal as well
    K2 = _rand(rng, 50, 64)
    assert np.allclose(A.attend_one(q, K2, V, 33, 0.0), V[:33].mean(axis=0),
                       rtol=1e-13, atol=1e-14)


def test_constant_values_give_the_constant():
    # the weights sum to one, seen through the output
    rng = np.random.default_rng(4)
    K = _rand(rng, 300, 64) * 8
    V = np.ones((300, 64))
    q = _rand(rng, 64)
    for n in (1, 2, 123, 300):
        assert np.allclose(A.attend_one(q, K, V, n, 0.125), 1.0, rtol=0, atol=1e-14)


def test_huge_score_gaps_select_the_best_key():
    # scores ~1e3 apart: exp without max-subtraction would overflow; the result is
    # the value row of the largest score
    rng = np.random.default_rng(5)
    K = _rand(rng, 200, 64)
    V = _rand(rng, 200, 64)
    q = _rand(rng, 64) * 4096
    s = K @ q
    j = int(np.argmax(s))
    gap = np.sort(s)[-1] - np.sort(s)[-2]
    assert gap * 0.125 > 50
    out = A.attend_one(q, K, V, 200, 0.125)
    assert np.all(np.isfinite(out))
    assert np.allclose(out, V[j], rtol=0, atol=1e-15)


def test_nonpositive_and_overlong_lengths():
    rng = np.random.default_rng(6)
    q = _rand(rng, 1, 1, 2, 64)
    K = _rand(rng, 1, 1, 2, 16, 64)
    V = _rand(rng, 1, 1, 2, 16, 64)
    for n in (0, -5):
        assert np.array_equal(A.attention(q, K, V, [n], 0.125, "f32"), np.zeros((1, 1, 2, 64)))
    a = A.attention(q, K, V, [1000], 0.125, "f32")
    b = A.attention(q, K, V, [16], 0.125, "f32")
    assert np.array_equal(a, b)


# -- invariants -------------------------------------------------------------------

def test_permuting_keys_and_values_together_changes_nothing():
    rng = np.random.default_rng(7)
    K = _rand(rng, 100, 64)
    V = _rand(rng, 100, 64)
    q = _rand(rng, 64)
    perm = rng.permutation(100)
    a = A.attend_one(q, K, V, 100, 0.125)
    b = A.attend_one(q, K[perm], V[perm], 100, 0.125)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-14)


def test_shifting_every_score_changes_nothing():
    rng = np.random.default_rng(8)
    K = _rand(rng, 100, 64)
    V = _rand(rng, 100, 64)
    q = _rand(rng, 64)
    shift = q / (q @ q) * 37.0            # adds 37 * scale to every score
    a = A.attend_one(q, K, V, 100, 0.125)
    b = A.attend_one(q, K + shift, V, 100, 0.125)
    assert np.allclose(a, b, rtol=1e-11, atol=1e-12)


def test_static_cache_with_mask_equals_dynamic_cache_and_ignores_invalid_slots():
    w = configs.TINY
    rng = np.random.default_rng(9)
    cap, n = 64, 29
    q = (rng.standard_normal((1, 1, 2, 64)) / 8).astype(np.float32)
    K = (rng.standard_normal((1, 1, 2, cap, 64)) / 8).astype(np.float32)
    V = (rng.standard_normal((1, 1, 2, cap, 64)) / 8).astype(np.float32)
    Kn, Vn = K.copy(), V.copy()
    Kn[..., n:, :] = np.nan
    Vn[..., n:, :] = np.inf
    static = A.attention(q, Kn, Vn, [n], w.scale, "f32")
    dynamic = A.attention(q, K[..., :n, :].copy(), V[..., :n, :].copy(), [n], w.scale, "f32")
    assert np.array_equal(static, dynamic)
    assert np.all(np.isfinite(static))


def test_bf16_path_equals_f32_path_on_the_decoded_values():
    rng = np.random.default_rng(10)
    qb = gen.f32_to_bf16_bits(rng.standard_normal((1, 1, 2, 64)).astype(np.float32))
    Kb = gen.f32_to_bf16_bits(rng.standard_normal((1, 1, 2, 20, 64)).astype(np.float32))
    Vb = gen.f32_to_bf16_bits(rng.standard_normal((1, 1, 2, 20, 64)).astype(np.float32))
    dec = lambda b: A.bf16_bits_to_f64(b).astype(np.float32)
    a = A.attention(qb, Kb, Vb, [13], 0.125, "bf16")
    b = A.attention(dec(qb), dec(Kb), dec(Vb), [13], 0.125, "f32")
    assert np.array_equal(a, b)


def test_rows_subset_matches_full():
    w = configs.TINY
    s_len, _ = gen.lengths(w)
    q = gen.queries(w, "self")
    K = gen.cache(w, "self", "k", s_len)
    V = gen.cache(w, "self", "v", s_len)
    full = A.attention(q, K, V, s_len, w.scale, w.dtype)
    rows = [(0, 0, 3), (0, 0, 1)]
    part = A.attention_rows(q, K, V, s_len, w.scale, w.dtype, rows)
    assert np.array_equal(part[0], full[0, 0, 3]) and np.array_equal(part[1], full[0, 0, 1])


def test_masked_attention_closed_forms_and_reductions():
    import math
    from oracle import attn as oa
    rng = np.random.default_rng(21)
    L, hd = 12, 8
    q = rng.standard_normal(hd)
    K = rng.standard_normal((L, hd))
    V = rng.standard_normal((L, hd))
    full = np.ones(L, bool)
    # all true: plain attention over the prefix
    for n in (1, 5, 12):
        assert np.allclose(oa.attend_masked(q, K, V, n, full, 0.3), oa.attend_one(q, K, V, n, 0.3))
    # a prefix mask equals a shorter length
    m = np.zeros(L, bool); m[:4] = True
    assert np.allclose(oa.attend_masked(q, K, V, 10, m, 0.3), oa.attend_one(q, K, V, 4, 0.3))
    # one attended key returns its value; none returns zeros; keys past n never count
    m = np.zeros(L, bool); m[7] = True
    assert np.array_equal(oa.attend_masked(q, K, V, 12, m, 0.3), V[7])
    assert not oa.attend_masked(q, K, V, 7, m, 0.3).any()
    # brute force with fsum over a scattered mask
    m = rng.random(L) < 0.5; m[2] = True
    keep = [j for j in range(9) if m[j]]
    s = [0.3 * math.fsum(q[d] * K[j, d] for d in range(hd)) for j in keep]
    mx = max(s); w = [math.exp(x - mx) for x in s]; Z = math.fsum(w)
    want = [math.fsum(w[i] * V[j, d] for i, j in enumerate(keep)) / Z for d in range(hd)]
    assert np.allclose(oa.attend_masked(q, K, V, 9, m, 0.3), want, rtol=1e-12, atol=1e-14)
    # permuting the keys together with the mask changes nothing
    p = rng.permutation(L)
    assert np.allclose(oa.attend_masked(q, K[p], V[p], L, m[p], 0.3),
                       oa.attend_masked(q, K, V, L, m, 0.3))


def test_round_bf16_matches_generator_rounding_and_ties():
    from oracle import attn as oa
    from workloads import gen
    x = np.random.default_rng(3).standard_normal(1000).astype(np.float32) * 100
    bits = gen.f32_to_bf16_bits(x)
    assert np.array_equal(oa.round_bf16(x).view(np.uint32), bits.astype(np.uint32) << 16)
    # ties to even: 1 + 2^-8 lies halfway between bf16 1 and 1 + 2^-7; even is 1
    assert oa.round_bf16(np.float32(1 + 2 ** -8)) == np.float32(1.0)
    assert oa.round_bf16(np.float32(1 + 3 * 2 ** -8)) == np.float32(1 + 2 ** -6)
