"""Pins for the sampler oracle (CPU only).

The kept set is checked against a stable library sort and a brute-force rank
count; the probabilities against scipy's softmax; the token against the
inverse-CDF definition (a deterministic sweep of u and a chi-square test of
sampled frequencies); plus closed forms and invariants.
"""
import math

import numpy as np
import pytest
from scipy import special, stats

from oracle import sampling as S
from workloads import configs, gen


def _brute_kept(x, k):
    # rank_i = number of entries that beat i (larger, or equal with a lower index)
    n = len(x)
    kk = min(k, n)
    kept = []
    for i in range(n):
        rank = sum(1 for j in range(n) if x[j] > x[i] or (x[j] == x[i] and j < i))
        if rank < kk:
            kept.append(i)
    return np.array(kept)


@pytest.mark.parametrize("seed", range(40))
def test_kept_set_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    x = rng.integers(-2, 3, size=n).astype(np.float64)   # many ties
    for k in range(1, 10):
        _, kept = S.kept_set(x, k)
        assert np.array_equal(kept, _brute_kept(x, k)), (x, k)


@pytest.mark.parametrize("seed", range(10))
def test_kept_set_matches_stable_argsort(seed):
    rng = np.random.default_rng(100 + seed)
    x = (rng.standard_normal(1089) * 3).astype(np.float32).astype(np.float64)
    x[rng.integers(0, 1089, 40)] = x[rng.integers(0, 1089, 40)]   # planted ties
    for k in (1, 2, 50, 64, 1089, 5000):
        ref = np.sort(np.argsort(-x, kind="stable")[:k])
        assert np.array_equal(S.kept_set(x, k)[1], ref)


@pytest.mark.parametrize("seed", range(10))
def test_probabilities_match_scipy_softmax(seed):
    rng = np.random.default_rng(200 + seed)
    x = (rng.standard_normal(1089) * 3).astype(np.float32).astype(np.float64)
    for k in (50, 250, 1089):
        for T in (0.05, 0.7, 1.0, 1.3, 25.0):
            tok, kept, p, C, _ = S.sample_row(x, T, k, 0.5)
            assert len(kept) == k
            ref = special.softmax(x[kept] / T)
            assert np.allclose(p, ref, rtol=1e-12, atol=1e-300)
            assert abs(math.fsum(p) - 1.0) < 1e-12
            assert tok in kept


@pytest.mark.parametrize("k", [50, 250])
def test_token_is_the_inverse_cdf_over_ascending_vocabulary(k):
    rng = np.random.default_rng(300)
    x = (rng.standard_normal(1089) * 3).astype(np.float32).astype(np.float64)
    T = 0.9
    _, kept, _, _, _ = S.sample_row(x, T, k, 0.0)
    p = special.softmax(x[kept] / T)
    bounds = [math.fsum(p[:r + 1]) for r in range(len(kept))]   # independent prefix sums
    # sweep u over a fine grid: the token must be kept[r] with bounds[r-1] <= u < bounds[r]
    for u in np.linspace(0.0, 1.0, 4001, endpoint=False):
        tok, _, _, C, dist = S.sample_row(x, T, k, float(u))
        r = next(i for i, b in enumerate(bounds) if u < b)
        if dist > 1e-12:
            assert tok == kept[r]


def test_chi_square_frequencies():
    rng = np.random.default_rng(400)
    x = np.array([0.3, -1.0, 2.0, 0.5, 1.5, -3.0, 0.0, 1.0])
    T, k = 0.8, 5
    _, kept, p, _, _ = S.sample_row(x, T, k, 0.0)
    n = 60000
    u = rng.random(n)
    counts = {int(i): 0 for i in kept}
    for ui in u:
        counts[S.sample_row(x, T, k, float(ui))[0]] += 1
    obs = np.array([counts[int(i)] for i in kept])
    chi2 = float(np.sum((obs - n * p) ** 2 / (n * p)))
    assert chi2 < stats.chi2.ppf(0.999, df=len(kept) - 1)


def test_two_element_closed_form():
    # k = 2 keeps the two largest; p(first kept) = sigmoid((x_a - x_b) / T)
    x = np.array([-5.0, 1.25, -7.0, 0.5, -9.0])
    T = 0.6
    _, kept, p, _, _ = S.sample_row(x, T, 2, 0.1)
    assert list(kept) == [1, 3]
    pa = 1.0 / (1.0 + math.exp(-(1.25 - 0.5) / T))
    assert abs(p[0] - pa) < 1e-15
    assert S.sample_row(x, T, 2, pa - 1e-9)[0] == 1
    assert S.sample_row(x, T, 2, pa + 1e-9)[0] == 3


def test_greedy_and_k1_are_argmax():
    rng = np.random.default_rng(500)
    for _ in range(50):
        x = rng.integers(-3, 4, size=30).astype(np.float64)   # ties: argmax takes the first
        want = int(np.argmax(x))
        for T in (0.0, -1.0):
            tok, kept, p, _, _ = S.sample_row(x, T, 10, float(rng.random()))
            assert tok == want and p.sum() == 1.0 and p[list(kept).index(want)] == 1.0
        for T in (0.5, 2.0):
            assert S.sample_row(x, T, 1, float(rng.random()))[0] == want


def test_invariants_shift_and_temperature():
    rng = np.random.default_rng(600)
    x = (rng.standard_normal(1089) * 3).astype(np.float64)
    for u in rng.random(20):
        t1, k1, p1, _, d1 = S.sample_row(x, 1.3, 50, u)
        t2, k2, p2, _, _ = S.sample_row(x + 1000.0, 1.3, 50, u)     # shift (exp range)
        t3, k3, p3, _, _ = S.sample_row(x / 1.3, 1.0, 50, u)        # fold T into x
        t4, k4, _, _, _ = S.sample_row(x, 0.2, 50, u)               # set independent of T
        assert np.array_equal(k1, k2) and np.array_equal(k1, k3) and np.array_equal(k1, k4)
        assert np.allclose(p1, p2, rtol=1e-12) and np.allclose(p1, p3, rtol=1e-12)
        if d1 > 1e-9:
            assert t1 == t2 == t3


def test_padding_is_never_a_candidate_and_rows_are_independent():
    w = configs.MINI_V1
    lg = gen.logits(w, pad_value=1e30)
    u = gen.uniforms(w)
    T = gen.temperatures(w)
    out = S.sample(lg, w.vocab_valid, T, w.top_k, u)
    assert np.all(out["tokens"] < w.vocab_valid)
    assert np.all(out["topk_idx"] < w.vocab_valid)
    for c in range(w.n_codebooks):
        tok = S.sample_row(lg[0, c, :w.vocab_valid].astype(np.float64), 1.0, 50, u[0, c])[0]
        assert tok == out["tokens"][0, c]


def test_k_larger_than_vocabulary_is_clamped():
    x = np.array([1.0, 3.0, 2.0])
    tok, kept, p, C, _ = S.sample_row(x, 1.0, 50, 0.99)
    assert list(kept) == [0, 1, 2]
    assert np.allclose(p, special.softmax(x))
    out = S.sample(x.reshape(1, 1, 3).astype(np.float32), 3, [1.0], 5, np.array([[0.2]]))
    assert list(out["topk_idx"][0, 0]) == [0, 1, 2, -1, -1]
    assert list(out["topk_prob"][0, 0, 3:]) == [0.0, 0.0]


def test_boundary_comparison_is_strict_and_overflow_takes_the_last():
    # two equal logits: p = [1/2, 1/2] exactly, C = [0.5, 1.0]
    x = np.array([0.0, 0.0])
    assert S.sample_row(x, 1.0, 2, 0.0)[0] == 0
    assert S.sample_row(x, 1.0, 2, np.nextafter(0.5, 0))[0] == 0
    assert S.sample_row(x, 1.0, 2, 0.5)[0] == 1          # u == C_0 goes to the next entry
    # u at or past the last boundary (only by caller error or rounding): last kept entry
    y = np.array([1.0, -4.0, 3.0, 2.0])
    assert S.sample_row(y, 1.0, 3, 1.0)[0] == 3
    assert S.sample_row(y, 1.0, 3, 7.5)[0] == 3


# ---- dist: the distance from u to the nearest CDF boundary ------------------------------
# It decides which token mismatches a GPU comparison may excuse (a uniform within the
# band of a boundary makes either neighbour correct under rounding), so it is pinned on
# hand-computed rows where every boundary is known exactly.

def test_dist_two_equal_logits():
    # x = [0, 0], T = 1, k = 2: p = [1/2, 1/2], boundaries C = [1/2, 1]
    x = np.zeros(2)
    for u, tok, dist in ((0.49, 0, 0.01), (0.5, 1, 0.0), (0.999, 1, 0.001), (0.0, 0, 0.5),
                         (0.75, 1, 0.25)):
        t, _, _, C, d = S.sample_row(x, 1.0, 2, u)
        assert np.allclose(C, [0.5, 1.0], rtol=0, atol=1e-15)
        assert t == tok and abs(d - dist) <= 1e-12, (u, t, d)


def test_dist_four_boundaries():
    # p proportional to 1, 2, 3, 4 (logits log 1 .. log 4): C = [0.1, 0.3, 0.6, 1.0]
    x = np.log(np.array([1.0, 2.0, 3.0, 4.0]))
    cases = ((0.05, 0, 0.05), (0.31, 2, 0.01), (0.29, 1, 0.01), (0.55, 2, 0.05),
             (0.61, 3, 0.01), (0.8, 3, 0.2), (0.97, 3, 0.03))
    for u, tok, dist in cases:
        t, S_, p, C, d = S.sample_row(x, 1.0, 4, u)
        assert np.allclose(p, [0.1, 0.2, 0.3, 0.4], rtol=0, atol=1e-15)
        assert np.allclose(C, [0.1, 0.3, 0.6, 1.0], rtol=0, atol=1e-15)
        assert t == tok and abs(d - dist) <= 1e-12, (u, t, d)


def test_dist_counts_only_the_kept_set_and_its_order():
    # vocabulary order [4, 1, 3, 2] scaled by log: kept (k = 3) = indices 0, 2, 3 with
    # weights 4, 3, 2 in ascending index order: C = [4/9, 7/9, 1]; index 1 is dropped
    x = np.log(np.array([4.0, 1.0, 3.0, 2.0]))
    t, kept, p, C, d = S.sample_row(x, 1.0, 3, 0.5)
    assert list(kept) == [0, 2, 3]
    assert np.allclose(C, [4 / 9, 7 / 9, 1.0], rtol=0, atol=1e-15)
    assert t == 2 and abs(d - (0.5 - 4 / 9)) <= 1e-12
    # temperature 2 flattens the weights to sqrt: 2, sqrt 3, sqrt 2
    w = np.sqrt([4.0, 3.0, 2.0])
    t, kept, p, C, d = S.sample_row(x, 2.0, 3, 0.5)
    Cw = np.cumsum(w) / w.sum()
    assert np.allclose(C, Cw, rtol=0, atol=1e-15)
    assert abs(d - np.min(np.abs(0.5 - Cw))) <= 1e-12


def test_dist_single_kept_entry_and_greedy():
    x = np.array([5.0, 0.0, 0.0, 0.0])
    t, _, _, C, d = S.sample_row(x, 1.0, 1, 0.3)
    assert t == 0 and list(C) == [1.0] and abs(d - 0.7) <= 1e-12
    t, _, _, _, d = S.sample_row(x, 0.0, 4, 0.3)
    assert t == 0 and d == np.inf                   # greedy rows have no boundary
