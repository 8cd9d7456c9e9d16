"""GPU parity of attention over a paged cache, through the C ABI.

The pool is built from the same seeded static cache: every sequence's logical blocks
are scattered over a shuffled pool (tails past the valid prefix and unused blocks hold
NaN, so any stray read shows).  Bars:
* paged == static bit for bit (same arithmetic, only addresses differ), in both the
  whole-sequence and the chunk-split schedule, for self-only and fused-step launches;
* against the oracle (rows gathered through the table) within the 2e-3 row bar;
* a table entry outside the pool reads as zero rows, matching the oracle with those
  rows zeroed.
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

BAR = 2e-3
LENS = [2049, 1, 64, 1025, 0, 65]


def _dev(a):
    return wdev.to_device(np.asarray(a), hp.DEV)


def _workload(B):
    return dataclasses.replace(configs.MINI_V1, n_layers=3, batch=B, self_cap=4096)


def _paged(static, lens, bs, extra_blocks, seed):
    """Scatter a static cache [NL, B, H, L, hd] into a pool; returns (pool, table)."""
    NL, B, H, L, hd = static.shape
    mb = L // bs
    nb = B * mb + extra_blocks
    rng = np.random.default_rng(seed)
    phys = rng.permutation(nb)[:B * mb].reshape(B, mb).astype(np.int32)
    pool = np.empty((NL, nb, H, bs, hd), static.dtype)
    pool[...] = gen.BF16_NAN if static.dtype == np.uint16 else np.float32(np.nan)
    for b in range(B):
        for i in range(mb):
            pool[:, phys[b, i]] = static[:, b, :, i * bs:(i + 1) * bs]
    return pool, phys


def _static_out(w, d, lens_d, ws):
    return hp.attn("self", w, d, ws=ws, lens=lens_d)


@pytest.mark.parametrize("bs", [64, 256, 4096])
@pytest.mark.parametrize("split", ["1", "0"])
def test_paged_self_equals_static_and_oracle(bs, split, tune):
    tune(attn_schedule=1 if split == "1" else 2)
    w = _workload(len(LENS))
    print(f"[paged] bs={bs} split={split} lens={LENS}", flush=True)
    d = wdev.step_inputs(w, hp.DEV, self_lens=LENS)
    lens_d = _dev(np.array(LENS, np.int32))
    ws = hp.workspace(w, w.self_cap, 0)
    want_static = hp.host(_static_out(w, d, lens_d, ws))
    ks = gen.cache(w, "self", "k", LENS)
    vs = gen.cache(w, "self", "v", LENS)
    kp, table = _paged(ks, LENS, bs, 7, seed=bs)
    vp, _ = _paged(vs, LENS, bs, 7, seed=bs)
    out = hp.out_buf(w)
    mb = w.self_cap // bs
    dec.dec_attn_self_paged(d["q_self"], _dev(kp), _dev(vp), _dev(table), lens_d, out,
                            w.n_layers, w.batch, w.heads, 64, bs, kp.shape[1], mb, dec.DEC_BF16,
                            w.scale, ws[0], ws[1])
    got = hp.host(out)
    assert np.array_equal(got.view(np.uint32), want_static.view(np.uint32)), \
        "paged differs from static"
    q = oattn.bf16_bits_to_f64(gen.queries(w, "self"))
    worst = 0.0
    for layer in range(w.n_layers):
        for b, n in enumerate(LENS):
            for h in range(w.heads):
                K = oattn.bf16_bits_to_f64(ocache.gather_paged(kp, table, bs, layer, b, h, n))
                V = oattn.bf16_bits_to_f64(ocache.gather_paged(vp, table, bs, layer, b, h, n))
                o = oattn.attend_one(q[layer, b, h], K, V, n, w.scale)
                worst = max(worst, hp.row_rel_err(got[layer, b, h], o))
    assert worst <= BAR, worst
    print(f"  max row rel err {worst:.2e}", flush=True)


def test_paged_step_equals_static_step():
    w = dataclasses.replace(_workload(2), cross_cap=64, cross_len=64)
    lens = [1500, 300]
    d = wdev.step_inputs(w, hp.DEV, self_lens=lens)
    ws = hp.workspace(w, w.self_cap, w.cross_cap)
    lens_d = _dev(np.array(lens, np.int32))
    d["len"] = lens_d
    o_s, o_c = hp.attn_step(w, d, ws=ws)
    bs = 128
    kp, table = _paged(gen.cache(w, "self", "k", lens), lens, bs, 3, seed=5)
    vp, _ = _paged(gen.cache(w, "self", "v", lens), lens, bs, 3, seed=5)
    p_s, p_c = hp.out_buf(w), hp.out_buf(w)
    dec.dec_attn_step_paged(d["q_self"], _dev(kp), _dev(vp), _dev(table), lens_d, bs,
                            kp.shape[1], w.self_cap // bs, p_s, d["q_cross"], d["k_cross"],
                            d["v_cross"], d["enc_len"], w.cross_cap, p_c, w.n_layers, w.batch,
                            w.heads, 64, dec.DEC_BF16, w.scale, ws[0], ws[1])
    for a, b in ((p_s, o_s), (p_c, o_c)):
        assert np.array_equal(hp.host(a).view(np.uint32), hp.host(b).view(np.uint32))


def test_out_of_pool_table_entry_reads_zero_rows():
    w = _workload(1)
    lens, bs = [300], 64
    d = wdev.step_inputs(w, hp.DEV, self_lens=lens)
    kp, table = _paged(gen.cache(w, "self", "k", lens), lens, bs, 2, seed=9)
    vp, _ = _paged(gen.cache(w, "self", "v", lens), lens, bs, 2, seed=9)
    nb = kp.shape[1]
    bad = table.copy()
    bad[0, 1] = -5          # keys 64..127
    bad[0, 3] = nb + 11     # keys 192..255
    ws = hp.workspace(w, w.self_cap, 0)
    out = hp.out_buf(w)
    dec.dec_attn_self_paged(d["q_self"], _dev(kp), _dev(vp), _dev(bad), _dev(np.array(lens, np.int32)),
                            out, w.n_layers, 1, w.heads, 64, bs, nb, w.self_cap // bs,
                            dec.DEC_BF16, w.scale, ws[0], ws[1])
    got = hp.host(out)
    assert np.all(np.isfinite(got))
    q = oattn.bf16_bits_to_f64(gen.queries(w, "self"))
    n = lens[0]
    for layer in range(w.n_layers):
        for h in range(w.heads):
            K = oattn.bf16_bits_to_f64(ocache.gather_paged(kp, table, bs, layer, 0, h, n))
            V = oattn.bf16_bits_to_f64(ocache.gather_paged(vp, table, bs, layer, 0, h, n))
            for blk in (1, 3):
                K[blk * bs:(blk + 1) * bs] = 0.0
                V[blk * bs:(blk + 1) * bs] = 0.0
            o = oattn.attend_one(q[layer, 0, h], K, V, n, w.scale)
            assert hp.row_rel_err(got[layer, 0, h], o) <= BAR


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("split", ["1", "0"])
def test_paged_widened_step_equals_static_widened_step(out, split, tune):
    # a paged self cache with a masked description and fp32 / bf16 outputs in one launch
    # (dec_attn_step_paged_ex) against the static widened step on the same keys
    tune(attn_schedule=1 if split == "1" else 2)
    w = dataclasses.replace(_workload(2), cross_cap=512, cross_len=None, cross_len_range=(1, 512))
    lens = [1500, 300]
    enc = np.array([512, 300], np.int32)
    print(f"[paged ex] out={out} split={split}", flush=True)
    d = wdev.step_inputs(w, hp.DEV, self_lens=lens, cross_lens=enc,
                         fill_lens=(np.array(lens), np.full(2, w.cross_cap)))
    lens_d = _dev(np.array(lens, np.int32))
    rng = np.random.default_rng(5)
    mask = rng.random((2, w.cross_cap)) < 0.4
    mask[:, 64:192] = False                   # whole tiles with no attended key
    words = 2 * ((w.cross_cap + 63) // 64)
    packed = np.zeros((2, words), np.uint32)
    for j in range(w.cross_cap):
        packed[:, j // 32] |= mask[:, j].astype(np.uint32) << np.uint32(j % 32)
    mask_d = _dev(packed)
    ws = hp.workspace(w, w.self_cap, w.cross_cap)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    ocode = dec.DEC_BF16 if out == "bf16" else dec.DEC_F32
    shape = (w.n_layers, 2, w.heads, 64)
    r_s, r_c = torch.empty(shape, dtype=odt, device=hp.DEV), torch.empty(shape, dtype=odt, device=hp.DEV)
    dec.dec_attn_step_ex(d["q_self"], d["k_self"], d["v_self"], lens_d, w.self_cap, r_s,
                         d["q_cross"], d["k_cross"], d["v_cross"], d["enc_len"], mask_d, words,
                         w.cross_cap, r_c, w.n_layers, 2, w.heads, 64, dec.DEC_BF16, ocode,
                         w.scale, ws[0], ws[1])
    bs = 128
    kp, table = _paged(gen.cache(w, "self", "k", lens), lens, bs, 3, seed=9)
    vp, _ = _paged(gen.cache(w, "self", "v", lens), lens, bs, 3, seed=9)
    p_s, p_c = torch.empty_like(r_s), torch.empty_like(r_c)
    dec.dec_attn_step_paged_ex(d["q_self"], _dev(kp), _dev(vp), _dev(table), lens_d, bs,
                               kp.shape[1], w.self_cap // bs, p_s, d["q_cross"], d["k_cross"],
                               d["v_cross"], d["enc_len"], mask_d, words, w.cross_cap, p_c,
                               w.n_layers, 2, w.heads, 64, dec.DEC_BF16, ocode, w.scale,
                               ws[0], ws[1])
    torch.cuda.synchronize()
    for a, b in ((p_s, r_s), (p_c, r_c)):
        va = a.view(torch.int16) if out == "bf16" else a.view(torch.int32)
        vb = b.view(torch.int16) if out == "bf16" else b.view(torch.int32)
        assert torch.equal(va, vb)
