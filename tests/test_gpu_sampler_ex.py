"""GPU parity of the widened sampler (dec_sample_topk_ex) against the oracle, through the C ABI.

* top_k > 64 (radix search over the row, or, for top_k <= 256, over the entries that pass a
  lower bound on the k-th key, compacted in vocabulary order; the CDF is one 64-lane scan per
  slot of 64 entries plus a running total, in float64): the bars of tests/sampler_check.py --
  sets exact; probabilities within half a float32 ulp; the sampled CDF within 2^-24 of the
  oracle's (and 5e-7) at every k and V; tokens exact outside the 1e-6 band.
* bf16 logits: each value widens exactly to float32, so the oracle reads the same widened
  values; the same bars.
* top_k <= 64 through the widened entry runs the standard kernel: tokens, sets and
  probabilities equal dec_sample_topk's bit for bit on fp32 logits; uniforms == NULL
  equals dec_sample_topk_philox bit for bit.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import autoregressive_audio_token_amd as dec  # noqa: E402
from oracle import sampling as osamp, rng as orng  # noqa: E402
from workloads import configs, gen, device as wdev  # noqa: E402
from tests import hip_path as hp, sampler_check  # noqa: E402



def _dev(a):
    return wdev.to_device(np.asarray(a), hp.DEV)


def _bf16_values(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _run(lg_d, dt, B, V, S, T, k, u, seed=0, step=None, fill=-1, n_cb=9):
    tokens = torch.full((B, n_cb), -7, dtype=torch.int32, device=hp.DEV)
    idx = torch.full((B, n_cb, k), -7, dtype=torch.int32, device=hp.DEV)
    prob = torch.full((B, n_cb, k), float("nan"), dtype=torch.float32, device=hp.DEV)
    dec.dec_sample_topk_ex(lg_d, dt, B, n_cb, V, S, _dev(T), k, None if u is None else _dev(u),
                           seed, None if step is None else _dev(step), fill, tokens, idx, prob)
    return hp.host(tokens), hp.host(idx), hp.host(prob)


def _compare(values, V, T, k, u, step, fill, got):
    tokens, idx, prob = got
    want = osamp.sample(values, V, T, k, u, step, fill)
    st = sampler_check.check(want, tokens, idx, prob, T, k, V)
    print(f"  rows={st['rows']} boundary_excluded={st['excluded']} prob_err={st['prob_err']:.2e} "
          f"cdf_err={st['cdf_err']:.2e}", flush=True)


def _logits(rng, B, V, scale=3.0, n_cb=9):
    S = V + (-V) % 8
    lg = np.full((B, n_cb, S), 1e30, np.float32)
    lg[:, :, :V] = rng.standard_normal((B, n_cb, V), dtype=np.float32) * np.float32(scale)
    return lg, S


@pytest.mark.parametrize("V", [65, 257, 1089, 3000, 4096])
@pytest.mark.parametrize("k", [65, 100, 250, 1024, 4096])
def test_wide_top_k_matches_oracle(V, k):
    rng = np.random.default_rng(V * 7 + k)
    B = 3
    print(f"[wide] V={V} k={k}", flush=True)
    lg, S = _logits(rng, B, V)
    T = np.array([1.0, 0.0, 0.5], np.float32)       # row 1 greedy
    u = rng.random((B, 9), dtype=np.float32)
    got = _run(_dev(lg), dec.DEC_F32, B, V, S, T, k, u)
    _compare(lg, V, T, k, u, None, -1, got)


def test_wide_many_rows_and_uniform_sweep():
    w = configs.MINI_V1
    B, k = 32, 250
    rng = np.random.default_rng(21)
    lg, S = _logits(rng, B, w.vocab_valid, scale=2.0)
    T = rng.uniform(0.7, 1.3, B).astype(np.float32)
    lg_d = _dev(lg)
    for rep in range(3):
        u = rng.random((B, 9), dtype=np.float32)
        got = _run(lg_d, dec.DEC_F32, B, w.vocab_valid, S, T, k, u, fill=1089)
        _compare(lg, w.vocab_valid, T, k, u, None, 1089, got)


def test_wide_ties_at_the_kth_value_keep_the_lowest_indices():
    B, V, k = 4, 1089, 300
    rng = np.random.default_rng(31)
    lg = np.full((B, 9, 1096), 1e30, np.float32)
    lg[:, :, :V] = np.round(rng.standard_normal((B, 9, V)) * 2).astype(np.float32)
    T = np.array([1.0, 0.7, -1.0, 2.0], np.float32)
    u = rng.random((B, 9), dtype=np.float32)
    got = _run(_dev(lg), dec.DEC_F32, B, V, 1096, T, k, u, fill=1089)
    _compare(lg, V, T, k, u, None, 1089, got)


def test_wide_delay_mask_and_greedy_first_maximum():
    B, V, k = 2, 1089, 500
    lg = np.zeros((B, 9, 1096), np.float32)
    lg[:, :, V:] = 1e30
    lg[:, :, 700] = 5.0
    lg[:, :, 1000] = 5.0               # tie at the maximum: the lower index wins
    T = np.array([0.0, 0.0], np.float32)
    u = np.full((B, 9), 0.5, np.float32)
    step = np.array([3, 20], np.int32)
    tokens, idx, prob = _run(_dev(lg), dec.DEC_F32, B, V, 1096, T, k, u, step=step, fill=1089)
    assert np.all(tokens[0, :4] == 700) and np.all(tokens[0, 4:] == 1089)
    assert np.all(tokens[1] == 700)
    # greedy probabilities: one-hot on the argmax, also where the fill token was emitted
    pos700 = np.argmax(idx == 700, axis=-1)
    assert np.all(prob[np.arange(B)[:, None], np.arange(9)[None, :], pos700] == 1.0)
    assert np.all(prob.sum(-1) == 1.0)


@pytest.mark.parametrize("k", [50, 64, 250])
def test_bf16_logits_match_oracle(k):
    w = configs.MINI_V1
    B = 4
    rng = np.random.default_rng(40 + k)
    bits = gen.f32_to_bf16_bits(rng.standard_normal((B, 9, 1096), dtype=np.float32) * 3)
    bits[:, :, w.vocab_valid:] = gen.BF16_NAN          # padding: never read
    values = _bf16_values(bits)
    T = np.array([1.0, 0.8, 0.0, 1.5], np.float32)
    u = rng.random((B, 9), dtype=np.float32)
    got = _run(_dev(bits), dec.DEC_BF16, B, w.vocab_valid, 1096, T, k, u, fill=1089)
    _compare(values, w.vocab_valid, T, k, u, None, 1089, got)


def test_narrow_k_is_the_standard_kernel():
    w = configs.MINI_V1
    B = 6
    rng = np.random.default_rng(50)
    lg, S = _logits(rng, B, w.vocab_valid)
    T = rng.uniform(0.5, 1.5, B).astype(np.float32)
    T[2] = 0.0
    u = rng.random((B, 9), dtype=np.float32)
    step = np.array([0, 1, 4, 8, 9, 100], np.int32)
    lg_d = _dev(lg)
    got = _run(lg_d, dec.DEC_F32, B, w.vocab_valid, S, T, w.top_k, u, step=step, fill=1089)
    ref = hp.sample(w, lg_d, _dev(T), _dev(u), step=_dev(step), B=B, fill=1089)
    for a, b in zip(got, ref):
        b = hp.host(b)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("k", [50, 250])
def test_null_uniforms_draw_philox(k):
    w = configs.MINI_V1
    B = 3
    rng = np.random.default_rng(60)
    lg, S = _logits(rng, B, w.vocab_valid)
    T = np.array([1.0, 0.9, 1.2], np.float32)
    step = np.array([11, 12, 500], np.int32)
    seed = 0x1234_5678_9ABC_DEF0
    lg_d = _dev(lg)
    got = _run(lg_d, dec.DEC_F32, B, w.vocab_valid, S, T, k, None, seed=seed, step=step, fill=1089)
    u = orng.sample_uniforms(seed, step.tolist(), 9).astype(np.float32)
    _compare(lg, w.vocab_valid, T, k, u, step, 1089, got)
    if k <= 64:
        tokens = torch.empty((B, 9), dtype=torch.int32, device=hp.DEV)
        idx = torch.empty((B, 9, k), dtype=torch.int32, device=hp.DEV)
        prob = torch.empty((B, 9, k), dtype=torch.float32, device=hp.DEV)
        dec.dec_sample_topk_philox(lg_d, B, 9, w.vocab_valid, S, _dev(T), k, seed, _dev(step),
                                   1089, tokens, idx, prob)
        for a, b in zip(got, (tokens, idx, prob)):
            assert np.array_equal(a.view(np.uint32), hp.host(b).view(np.uint32))


def test_wide_nonfinite_logits_still_give_a_valid_index():
    B, V, k = 2, 1089, 200
    rng = np.random.default_rng(9)
    lg = (rng.standard_normal((B, 9, 1096)) * 3).astype(np.float32)
    lg[0, :, ::7] = np.nan
    lg[1, :, ::5] = np.inf
    lg[1, 3, :] = -np.inf
    T = np.array([1.0, 1.0], np.float32)
    u = rng.random((B, 9), dtype=np.float32)
    tokens, idx, _ = _run(_dev(lg), dec.DEC_F32, B, V, 1096, T, k, u)
    assert np.all((tokens >= 0) & (tokens < V))
    assert np.all((idx >= 0) & (idx < V))


@pytest.mark.parametrize("V,k", [(1089, 65), (1089, 200), (4096, 128), (4096, 256)])
def test_wide_pruned_rows_with_heavy_ties(V, k):
    # top_k in the pruned range: values on a few levels, so many entries tie at the k-th
    # key (all survive the bound; the lowest indices are kept), and flat rows whose
    # survivors overflow the pruned capacity (the whole row is searched instead)
    B = 4
    rng = np.random.default_rng(V + k)
    S = V + (-V) % 8
    lg = np.full((B, 9, S), 1e30, np.float32)
    lg[:, :, :V] = np.round(rng.standard_normal((B, 9, V)) * 1.5).astype(np.float32)
    lg[3, :4, :V] = 0.5                      # flat rows
    lg[3, 4:, :V] = np.round(rng.random((5, V)) * 2).astype(np.float32)   # three levels
    T = np.array([1.0, 0.6, 0.0, 1.4], np.float32)
    u = rng.random((B, 9), dtype=np.float32)
    print(f"[wide pruned ties] V={V} k={k}", flush=True)
    got = _run(_dev(lg), dec.DEC_F32, B, V, S, T, k, u, fill=1089)
    _compare(lg, V, T, k, u, None, 1089, got)
