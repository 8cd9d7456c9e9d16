"""GPU parity of the fused sampler against the oracle, through the C ABI.

Bars (tests/sampler_check.py): top-k index sets bit-exact; each probability within
half a float32 ulp of the oracle's; the CDF the kernel samples from (the float64
running sum of the probabilities it exports) within 2^-24 of the oracle's and within
5e-7; tokens exact except rows whose uniform lies within 1e-6 of an oracle CDF
boundary, at most max(2, rows / 1000) such rows.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

from oracle import sampling as osamp  # noqa: E402
from workloads import configs, gen, device as wdev  # noqa: E402
from tests import hip_path as hp, sampler_check  # noqa: E402



def _dev(a, dtype=None):
    return wdev.to_device(np.asarray(a), hp.DEV, dtype)


def _compare(logits, V_valid, T, k, u, step, fill, tokens, idx, prob):
    want = osamp.sample(logits, V_valid, T, k, u, step, fill)
    st = sampler_check.check(want, hp.host(tokens), hp.host(idx), hp.host(prob), T, k, V_valid)
    print(f"  rows={st['rows']} boundary_excluded={st['excluded']} prob_err={st['prob_err']:.2e} "
          f"cdf_err={st['cdf_err']:.2e}", flush=True)
    return want


@pytest.mark.parametrize("name", ["tiny", "mini_v1", "batched_mixed"])
def test_parity_workload(name):
    w = configs.BY_NAME[name]
    lg, u, T = gen.logits(w), gen.uniforms(w), gen.temperatures(w)
    tokens, idx, prob = hp.sample(w, _dev(lg), _dev(T), _dev(u))
    _compare(lg, w.vocab_valid, T, w.top_k, u, None, w.fill_token, tokens, idx, prob)


def test_parity_many_rows_and_uniform_sweep():
    # 64 sequences x 9 codebooks, several draws of the uniforms
    w = configs.MINI_V1
    B = 64
    rng = np.random.default_rng(11)
    lg = np.full((B, 9, w.vocab_stride), 1e30, np.float32)
    lg[:, :, :w.vocab_valid] = rng.standard_normal((B, 9, w.vocab_valid), dtype=np.float32) * 3
    T = rng.uniform(0.7, 1.3, B).astype(np.float32)
    for rep in range(4):
        u = rng.random((B, 9), dtype=np.float32)
        tokens, idx, prob = hp.sample(w, _dev(lg), _dev(T), _dev(u), B=B)
        _compare(lg, w.vocab_valid, T, w.top_k, u, None, 1089, tokens, idx, prob)


def test_delay_mask_long_output_steps():
    w = configs.LONG_OUTPUT
    for s in list(range(10)) + [128, 2047]:
        lg, u, T = gen.logits(w, s), gen.uniforms(w, s), gen.temperatures(w)
        step = np.array([s], np.int32)
        tokens, idx, prob = hp.sample(w, _dev(lg), _dev(T), _dev(u), step=_dev(step))
        _compare(lg, w.vocab_valid, T, w.top_k, u, step, w.fill_token, tokens, idx, prob)
        toks = hp.host(tokens)
        for c in range(9):
            assert (toks[0, c] == w.fill_token) == (s < c)


@pytest.mark.parametrize("V", [1, 2, 50, 63, 64, 65, 256, 257, 1024, 1089, 2048, 3000, 4096])
@pytest.mark.parametrize("k", [1, 50, 64])
def test_vocab_sizes_and_k(V, k):
    w = configs.MINI_V1
    rng = np.random.default_rng(V * 100 + k)
    B = 3
    stride = V + (-V) % 8
    lg = np.full((B, 9, stride), 1e30, np.float32)
    lg[:, :, :V] = rng.standard_normal((B, 9, V), dtype=np.float32) * 3
    T = np.array([1.0, 0.0, 0.5], np.float32)      # row 1 greedy
    u = rng.random((B, 9), dtype=np.float32)
    tokens, idx, prob = hp.sample(w, _dev(lg), _dev(T), _dev(u), top_k=k, V_valid=V, B=B)
    _compare(lg, V, T, k, u, None, -1, tokens, idx, prob)


def test_ties_at_the_kth_value_keep_the_lowest_indices():
    w = configs.MINI_V1
    B, V, k = 4, 1089, 50
    rng = np.random.default_rng(3)
    lg = np.full((B, 9, 1096), 1e30, np.float32)
    lg[:, :, :V] = np.round(rng.standard_normal((B, 9, V)) * 2).astype(np.float32)  # ~13 values
    T = np.array([1.0, 0.7, -1.0, 2.0], np.float32)
    u = rng.random((B, 9), dtype=np.float32)
    tokens, idx, prob = hp.sample(w, _dev(lg), _dev(T), _dev(u), B=B)
    _compare(lg, V, T, k, u, None, 1089, tokens, idx, prob)


def test_greedy_and_k1_pick_the_first_maximum():
    w = configs.MINI_V1
    B = 2
    lg = np.zeros((B, 9, 1096), np.float32)
    lg[:, :, 1089:] = 1e30
    lg[:, :, 100] = 5.0
    lg[:, :, 900] = 5.0          # tie at the maximum: the lower index wins
    T = np.array([0.0, 1.0], np.float32)
    u = np.full((B, 9), 0.999, np.float32)
    tokens, _, _ = hp.sample(w, _dev(lg), _dev(T), _dev(u), B=B)
    assert np.all(hp.host(tokens)[0] == 100)
    tokens, _, _ = hp.sample(w, _dev(lg), _dev(T), _dev(u), B=B, top_k=1)
    assert np.all(hp.host(tokens) == 100)


def test_nonfinite_logits_still_give_a_valid_index():
    w = configs.MINI_V1
    B = 2
    rng = np.random.default_rng(9)
    lg = (rng.standard_normal((B, 9, 1096)) * 3).astype(np.float32)
    lg[0, :, ::7] = np.nan
    lg[1, :, ::5] = np.inf
    lg[1, 3, :] = -np.inf
    T = np.array([1.0, 1.0], np.float32)
    u = rng.random((B, 9), dtype=np.float32)
    tokens, _, _ = hp.sample(w, _dev(lg), _dev(T), _dev(u), B=B)
    t = hp.host(tokens)
    assert np.all((t >= 0) & (t < w.vocab_valid))
