"""GPU parity on seeded random shapes, through the C ABI: attention and the sampler.

Each case draws its own shape, dtype, head dim, lengths (0, 1, the capacity, past the
capacity and negative included), entry point and schedule, and checks sampled output
rows against the oracle with the same bars as the targeted tests:
* attention: 2e-3 relative per row (max-norm), plus 2^-8 (half an ulp) when the outputs
  are bf16; sequences with no valid key exactly zero;
* sampler: top-k sets exact, tokens exact outside the 1e-6 band of a CDF boundary,
  probabilities and running sums within 1e-6 (top_k <= 64) or 2e-6 (wider; the
  derivation is in test_gpu_sampler_ex.py).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import autoregressive_audio_token_amd as dec  # noqa: E402
from oracle import attn as oattn, sampling as osamp, rng as orng  # noqa: E402
from workloads import configs, gen, device as wdev  # noqa: E402
from tests import hip_path as hp, sampler_check  # noqa: E402
from tests.oracle_inputs import RowSource, sampled_rows  # noqa: E402

BAR = 2e-3


def _dev(a):
    return wdev.to_device(np.asarray(a), hp.DEV)


def _lengths(rng, B, cap):
    n = rng.integers(0, cap + 1, B)
    for b in range(B):                       # edge cases mixed in
        u = rng.random()
        if u < 0.1:
            n[b] = 0
        elif u < 0.2:
            n[b] = 1
        elif u < 0.3:
            n[b] = cap
        elif u < 0.35:
            n[b] = cap + int(rng.integers(1, 100))   # read as cap
        elif u < 0.4:
            n[b] = -int(rng.integers(1, 5))         # no valid key
    return n.astype(np.int32)


def _attention_case(seed):
    rng = np.random.default_rng(seed)
    hd = int(rng.choice([64, 128]))
    w = configs.Workload(
        cfg_id=300 + seed, name=f"random{seed}", n_layers=int(rng.integers(1, 4)),
        batch=int(rng.integers(1, 13)), heads=int(rng.integers(1, 7)), head_dim=hd,
        dtype=str(rng.choice(["bf16", "f32"])), self_cap=int(rng.integers(1, 2600)),
        cross_cap=int(rng.integers(1, 1300)), self_len=None, cross_len=None,
        self_len_range=(0, 1), cross_len_range=(0, 1), qkv_std=hd ** -0.5,
        cross_kv_std=hd ** -0.5, scale=hd ** -0.5)
    return rng, w


@pytest.mark.parametrize("seed", range(16))
def test_attention_random_shapes(seed, tune):
    rng, w = _attention_case(seed)
    s_len, c_len = _lengths(rng, w.batch, w.self_cap), _lengths(rng, w.batch, w.cross_cap)
    entry = str(rng.choice(["self", "cross", "step", "ex"]))
    split = str(rng.choice(["auto", "0", "1"]))
    if split != "auto":
        tune(attn_schedule=1 if split == "1" else 2)
    print(f"[random attn] seed={seed} NL={w.n_layers} B={w.batch} H={w.heads} hd={w.head_dim} "
          f"{w.dtype} caps=({w.self_cap},{w.cross_cap}) entry={entry} split={split}", flush=True)
    d = wdev.step_inputs(w, hp.DEV, self_lens=s_len, cross_lens=c_len)
    fill = (np.clip(s_len, 0, w.self_cap), np.clip(c_len, 0, w.cross_cap))
    src = RowSource(w, *fill)
    rows = sampled_rows(w, min(32, w.n_layers * w.batch * w.heads), seed=seed)
    ws = hp.workspace(w, w.self_cap, w.cross_cap)
    checks = []
    bf16_out = False
    if entry in ("self", "cross"):
        checks.append((entry, hp.attn(entry, w, d, ws=ws), None))
    elif entry == "step":
        o_s, o_c = hp.attn_step(w, d, ws=ws)
        checks += [("self", o_s, None), ("cross", o_c, None)]
    else:
        words = 2 * ((w.cross_cap + 63) // 64)
        mask = rng.random((w.batch, w.cross_cap)) < rng.uniform(0.2, 1.0)
        packed = np.zeros((w.batch, words), np.uint32)
        for j in range(w.cross_cap):
            packed[:, j // 32] |= mask[:, j].astype(np.uint32) << np.uint32(j % 32)
        bf16_out = bool(rng.random() < 0.5)
        odt = torch.bfloat16 if bf16_out else torch.float32
        shape = (w.n_layers, w.batch, w.heads, w.head_dim)
        o_s, o_c = torch.empty(shape, dtype=odt, device=hp.DEV), torch.empty(shape, dtype=odt, device=hp.DEV)
        dec.dec_attn_step_ex(d["q_self"], d["k_self"], d["v_self"], d["len"], w.self_cap, o_s,
                             d["q_cross"], d["k_cross"], d["v_cross"], d["enc_len"], _dev(packed),
                             words, w.cross_cap, o_c, w.n_layers, w.batch, w.heads, w.head_dim,
                             hp.code(w), dec.DEC_BF16 if bf16_out else dec.DEC_F32, w.scale,
                             ws[0], ws[1])
        checks += [("self", o_s.float(), None), ("cross", o_c.float(), mask)]
    for kind, out, mask in checks:
        got = hp.host(out)
        lens = s_len if kind == "self" else c_len
        if mask is None:
            want = src.expected(kind, lens, rows)
        else:
            want = np.zeros((len(rows), w.head_dim))
            q = src.q["cross"]
            dec16 = oattn.bf16_bits_to_f64 if w.dtype == "bf16" else (lambda x: np.asarray(x, np.float64))
            for i, (layer, b, h) in enumerate(rows):
                n = min(int(lens[b]), w.cross_cap)
                if n > 0:
                    K = dec16(src.kv("cross", "k", layer, b)[h])
                    V = dec16(src.kv("cross", "v", layer, b)[h])
                    want[i] = oattn.attend_masked(dec16(q[layer, b, h]), K, V, n, mask[b], w.scale)
        g = np.stack([got[layer, b, h] for layer, b, h in rows])
        assert np.all(np.isfinite(g))
        # bf16 outputs add their own rounding: at most half an ulp, 2^-8 of the value
        bar = BAR + (2.0 ** -8 if entry == "ex" and bf16_out else 0.0)
        err = hp.row_rel_err(g, want)
        print(f"  {kind}: max_rel_err={err:.3e}", flush=True)
        assert err <= bar, (kind, err)
        for i, (layer, b, h) in enumerate(rows):
            n = min(int(lens[b]), w.cross_cap if kind == "cross" else w.self_cap)
            if n <= 0 or (mask is not None and not mask[b, :n].any()):
                assert not g[i].any(), "a sequence with no valid key must give zeros"


@pytest.mark.parametrize("seed", range(24))
def test_sampler_random_shapes(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 41))
    n_cb = int(rng.integers(1, 13))
    V = int(rng.choice([int(rng.integers(1, 130)), int(rng.integers(130, 4097))]))
    S = V + int(rng.integers(0, 9))
    k = int(min(4096, rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, max(66, V + 21)))])))
    bf16 = bool(rng.random() < 0.3)
    ties = bool(rng.random() < 0.3)
    philox = bool(rng.random() < 0.3)
    print(f"[random sampler] seed={seed} B={B} n_cb={n_cb} V={V} S={S} k={k} bf16={bf16} "
          f"ties={ties} philox={philox}", flush=True)
    x = rng.standard_normal((B, n_cb, S), dtype=np.float32) * np.float32(rng.uniform(0.5, 5))
    if ties:
        x = np.round(x)
    x[:, :, V:] = 1e30                                   # padding: never a candidate
    if bf16:
        bits = gen.f32_to_bf16_bits(x)
        values = (bits.astype(np.uint32) << 16).view(np.float32)
        lg_d = _dev(bits)
    else:
        values = x
        lg_d = _dev(x)
    T = rng.uniform(0.3, 2.0, B).astype(np.float32)
    T[rng.random(B) < 0.2] = 0.0                         # greedy rows
    step = rng.integers(0, 12, B).astype(np.int32) if rng.random() < 0.5 else None
    seed_rng = int(rng.integers(0, 2 ** 63))
    if philox:
        steps = step.tolist() if step is not None else [0] * B
        u = orng.sample_uniforms(seed_rng, steps, n_cb).astype(np.float32)
        u_d = None
    else:
        u = rng.random((B, n_cb), dtype=np.float32)
        u_d = _dev(u)
    tokens = torch.full((B, n_cb), -7, dtype=torch.int32, device=hp.DEV)
    idx = torch.full((B, n_cb, k), -7, dtype=torch.int32, device=hp.DEV)
    prob = torch.full((B, n_cb, k), float("nan"), dtype=torch.float32, device=hp.DEV)
    dec.dec_sample_topk_ex(lg_d, dec.DEC_BF16 if bf16 else dec.DEC_F32, B, n_cb, V, S, _dev(T), k,
                           u_d, seed_rng, None if step is None else _dev(step), 4242, tokens, idx,
                           prob)
    tokens, idx, prob = hp.host(tokens), hp.host(idx), hp.host(prob)
    want = osamp.sample(values, V, T, k, u, step, 4242)
    sampler_check.check(want, tokens, idx, prob, T, k, V)
