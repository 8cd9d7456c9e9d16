"""GPU parity of attention at head dim 128, through the C ABI.

At head dim 128 a tile is 16 keys of 256 bytes (the bytes of a 32-key tile at head
dim 64), a chunk is 16 tile rounds, a score reduces over 16 lanes (bf16) or 32 (fp32),
and short sequences pack at most two to a workgroup.  Bars as at head dim 64:
* every output row within 2e-3 relative (max-norm) of the oracle, and within 1e-4 at
  these moderate score magnitudes (an fp32 dot product of 128 terms and an online
  softmax over at most 4096 keys stay far below it);
* the whole-sequence and the chunk-split schedules bit-equal;
* paged == static bit for bit;
* a key mask and bf16 outputs as in the head-dim-64 widening.
"""
import dataclasses

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import autoregressive_audio_token_amd as dec  # noqa: E402
from oracle import attn as oattn, cache as ocache  # noqa: E402
from workloads import configs, gen, device as wdev  # noqa: E402
from tests import hip_path as hp  # noqa: E402
from tests.oracle_inputs import RowSource, all_rows, sampled_rows  # noqa: E402

BAR = 2e-3
TIGHT = 1e-4
HD = 128


def _w(base=configs.MINI_V1, **kw):
    # same model width (16 heads of 64 = 8 heads of 128); q, k, v ~ N(0, 1/sqrt(128))
    return dataclasses.replace(base, heads=base.heads // 2, head_dim=HD, scale=HD ** -0.5,
                               qkv_std=HD ** -0.5, **kw)


def _dev(a):
    return wdev.to_device(np.asarray(a), hp.DEV)


def _inputs(w, **kw):
    print(f"[hd128] workload={w.name} dtype={w.dtype} heads={w.heads} {kw}", flush=True)
    return wdev.step_inputs(w, hp.DEV, **kw)


def _check(kind, w, out, src, rows, lens, tight=True):
    got = hp.host(out)
    want = src.expected(kind, lens, rows)
    g = np.stack([got[layer, b, h] for layer, b, h in rows])
    assert np.all(np.isfinite(g)), "non-finite output: an invalid (NaN) slot was read"
    err = hp.row_rel_err(g, want)
    print(f"  {kind}: rows={len(rows)} max_rel_err={err:.3e}", flush=True)
    assert err <= BAR
    if tight:
        assert err <= TIGHT
    return err


@pytest.mark.parametrize("base", ["tiny", "mini_v1", "long_description"])
def test_parity_full(base):
    w = _w(configs.BY_NAME[base])
    d = _inputs(w)
    s_len, c_len = d["self_len_host"], d["cross_len_host"]
    src = RowSource(w, s_len, c_len)
    rows = all_rows(w)
    _check("self", w, hp.attn("self", w, d), src, rows, s_len)
    _check("cross", w, hp.attn("cross", w, d), src, rows, c_len)
    o_s, o_c = hp.attn_step(w, d)
    _check("self", w, o_s, src, rows, s_len)
    _check("cross", w, o_c, src, rows, c_len)


@pytest.mark.parametrize("n", [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 1023, 1024,
                               1025, 2049, 4095, 4096])
@pytest.mark.parametrize("split", ["1", "0"])
def test_ragged_lengths_both_schedules(n, split, tune):
    tune(attn_schedule=1 if split == "1" else 2)
    w = _w(n_layers=4)
    lens = np.array([n], dtype=np.int32)
    d = _inputs(w, self_lens=lens)
    src = RowSource(w, lens, d["cross_len_host"])
    rows = sampled_rows(w, 24, seed=n)
    _check("self", w, hp.attn("self", w, d), src, rows, lens)


def test_schedules_are_bit_equal_and_batched_packing(tune):
    # 32 sequences of mixed lengths: short ones pack two to a workgroup
    w = _w(configs.BATCHED, n_layers=2)
    rng = np.random.default_rng(3)
    s_len = rng.integers(1, 2049, w.batch).astype(np.int32)
    s_len[:6] = [1, 2, 31, 32, 33, 64]
    d = _inputs(w, self_lens=s_len)
    ws = hp.workspace(w, w.self_cap, w.cross_cap)
    outs = []
    for split in ("1", "0"):
        tune(attn_schedule=1 if split == "1" else 2)
        outs.append([hp.host(o) for o in hp.attn_step(w, d, ws=ws)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    src = RowSource(w, s_len, d["cross_len_host"])
    rows = sampled_rows(w, 96, seed=9) + [(0, b, 0) for b in range(6)]
    _check("self", w, torch.from_numpy(outs[0][0]), src, rows, s_len)
    _check("cross", w, torch.from_numpy(outs[0][1]), src, rows, d["cross_len_host"])


def test_single_key_and_constant_values():
    w = _w()
    d = _inputs(w, self_lens=[1])
    out = hp.host(hp.attn("self", w, d))
    v0 = d["v_self"][:, :, :, 0, :].float().cpu().numpy()
    assert np.array_equal(out, v0)
    d = _inputs(w, self_lens=[777])
    d["v_self"].fill_(1.0)
    assert np.array_equal(hp.host(hp.attn("self", w, d)), np.ones((w.n_layers, 1, w.heads, HD),
                                                                   np.float32))


def _paged(static, bs, extra_blocks, seed):
    NL, B, H, L, hd = static.shape
    mb = L // bs
    nb = B * mb + extra_blocks
    rng = np.random.default_rng(seed)
    phys = rng.permutation(nb)[:B * mb].reshape(B, mb).astype(np.int32)
    pool = np.empty((NL, nb, H, bs, hd), static.dtype)
    pool[...] = gen.BF16_NAN
    for b in range(B):
        for i in range(mb):
            pool[:, phys[b, i]] = static[:, b, :, i * bs:(i + 1) * bs]
    return pool, phys


@pytest.mark.parametrize("split", ["1", "0"])
def test_paged_equals_static(split, tune):
    tune(attn_schedule=1 if split == "1" else 2)
    w = _w(n_layers=3, batch=4)
    lens = [2049, 33, 64, 0]
    d = _inputs(w, self_lens=lens)
    lens_d = _dev(np.array(lens, np.int32))
    ws = hp.workspace(w, w.self_cap, 0)
    want = hp.host(hp.attn("self", w, d, ws=ws, lens=lens_d))
    bs = 64
    kp, table = _paged(gen.cache(w, "self", "k", lens), bs, 5, seed=1)
    vp, _ = _paged(gen.cache(w, "self", "v", lens), bs, 5, seed=1)
    out = hp.out_buf(w)
    dec.dec_attn_self_paged(d["q_self"], _dev(kp), _dev(vp), _dev(table), lens_d, out,
                            w.n_layers, w.batch, w.heads, HD, bs, kp.shape[1], w.self_cap // bs,
                            dec.DEC_BF16, w.scale, ws[0], ws[1])
    got = hp.host(out)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "paged differs from static"
    q = oattn.bf16_bits_to_f64(gen.queries(w, "self"))
    worst = 0.0
    for layer in range(w.n_layers):
        for b, n in enumerate(lens):
            for h in range(w.heads):
                K = oattn.bf16_bits_to_f64(ocache.gather_paged(kp, table, bs, layer, b, h, n))
                V = oattn.bf16_bits_to_f64(ocache.gather_paged(vp, table, bs, layer, b, h, n))
                worst = max(worst, hp.row_rel_err(got[layer, b, h],
                                                  oattn.attend_one(q[layer, b, h], K, V, n, w.scale)))
    assert worst <= BAR, worst


def _pack(mask):
    B, L = mask.shape
    out = np.zeros((B, 2 * ((L + 63) // 64)), np.uint32)
    for j in range(L):
        out[:, j // 32] |= mask[:, j].astype(np.uint32) << np.uint32(j % 32)
    return out


@pytest.mark.parametrize("split", ["1", "0"])
def test_cross_mask_and_bf16_outputs(split, tune):
    tune(attn_schedule=1 if split == "1" else 2)
    B = 3
    w = _w(n_layers=2, batch=B, cross_cap=512, cross_len=None, cross_len_range=(1, 512),
           self_len=100)
    enc = np.array([512, 300, 77], np.int32)
    d = _inputs(w, cross_lens=enc, fill_lens=(np.full(B, 100), np.full(B, w.cross_cap)))
    rng = np.random.default_rng(12)
    mask = rng.random((B, w.cross_cap)) < 0.4
    mask[2, :] = False                  # no attended key: zeros
    mask[1, 300:] = True                # bits past enc_len: ignored
    mask[:, 32:96] = False              # whole 16-key tiles: not read (NaN there)
    for name in ("k_cross", "v_cross"):
        d[name][:, :, :, 32:96, :] = float("nan")
    packed = _pack(mask)
    ws = hp.workspace(w, w.self_cap, w.cross_cap)
    o_s, o_c = hp.out_buf(w), hp.out_buf(w)
    args = (d["q_self"], d["k_self"], d["v_self"], d["len"], w.self_cap)
    cross = (d["q_cross"], d["k_cross"], d["v_cross"], d["enc_len"])
    dec.dec_attn_step_ex(*args, o_s, *cross, _dev(packed), packed.shape[1], w.cross_cap, o_c,
                         w.n_layers, B, w.heads, HD, dec.DEC_BF16, dec.DEC_F32, w.scale,
                         ws[0], ws[1])
    got = hp.host(o_c)
    q = oattn.bf16_bits_to_f64(gen.queries(w, "cross"))
    worst = 0.0
    for layer in range(w.n_layers):
        for b in range(B):
            K = oattn.bf16_bits_to_f64(gen.kv_rows(w, "cross", "k", layer, b, w.cross_cap))
            V = oattn.bf16_bits_to_f64(gen.kv_rows(w, "cross", "v", layer, b, w.cross_cap))
            for h in range(w.heads):
                o = oattn.attend_masked(q[layer, b, h], K[h], V[h], enc[b], mask[b], w.scale)
                worst = max(worst, hp.row_rel_err(got[layer, b, h], o))
    assert worst <= BAR, worst
    assert not got[:, 2].any()
    # bf16 outputs: the fp32 outputs rounded to nearest even
    b_s = torch.empty((w.n_layers, B, w.heads, HD), dtype=torch.bfloat16, device=hp.DEV)
    b_c = torch.empty_like(b_s)
    dec.dec_attn_step_ex(*args, b_s, *cross, _dev(packed), packed.shape[1], w.cross_cap, b_c,
                         w.n_layers, B, w.heads, HD, dec.DEC_BF16, dec.DEC_BF16, w.scale,
                         ws[0], ws[1])
    for bf, f32 in ((b_s, o_s), (b_c, o_c)):
        want = oattn.round_bf16(hp.host(f32)).view(np.uint32) >> 16
        assert np.array_equal(bf.view(torch.int16).cpu().numpy().view(np.uint16),
                              want.astype(np.uint16))
