"""GPU parity of the widened attention entry point (dec_attn_step_ex), through the C ABI.

* bf16 outputs are the fp32 outputs rounded to nearest-even, bit for bit (the fp32
  outputs themselves are held to the oracle elsewhere);
* a boolean cross mask: an all-true mask changes no bit; random masks match the oracle
  within the 2e-3 row bar in both schedules; a row with no attended key is zero; bits
  past enc_len are ignored.
Masked keys below enc_len are still read (their weight is exactly zero), so they hold
finite values here, as in any real description cache.
"""
import dataclasses

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import autoregressive_audio_token_amd as dec  # noqa: E402
from oracle import attn as oattn  # noqa: E402
from workloads import configs, gen, device as wdev  # noqa: E402
from tests import hip_path as hp  # noqa: E402

BAR = 2e-3


def _dev(a):
    return wdev.to_device(np.asarray(a), hp.DEV)


def _pack(mask):
    """[B, L] bool -> [B, words] uint32 (bit j % 32 of word j // 32), words even."""
    B, L = mask.shape
    words = 2 * ((L + 63) // 64)
    out = np.zeros((B, words), np.uint32)
    for j in range(L):
        out[:, j // 32] |= mask[:, j].astype(np.uint32) << np.uint32(j % 32)
    return out


def _ex(w, d, out_s, out_c, ws, mask=None, words=0, out_dtype=None):
    dec.dec_attn_step_ex(d["q_self"], d["k_self"], d["v_self"], d["len"], w.self_cap, out_s,
                         d["q_cross"], d["k_cross"], d["v_cross"], d["enc_len"], mask, words,
                         w.cross_cap, out_c, w.n_layers, w.batch, w.heads, 64, hp.code(w),
                         dec.DEC_F32 if out_dtype is None else out_dtype, w.scale, ws[0], ws[1])


@pytest.mark.parametrize("name", ["mini_v1", "long_description", "tiny"])
def test_bf16_outputs_are_the_rounded_fp32_outputs(name):
    w = configs.BY_NAME[name]
    d = wdev.step_inputs(w, hp.DEV)
    ws = hp.workspace(w, w.self_cap, w.cross_cap)
    o_s, o_c = hp.attn_step(w, d, ws=ws)
    b_s = torch.empty((w.n_layers, w.batch, w.heads, 64), dtype=torch.bfloat16, device=hp.DEV)
    b_c = torch.empty_like(b_s)
    _ex(w, d, b_s, b_c, ws, out_dtype=dec.DEC_BF16)
    for got, f32 in ((b_s, o_s), (b_c, o_c)):
        want = oattn.round_bf16(hp.host(f32)).view(np.uint32) >> 16
        got_bits = got.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got_bits, want.astype(np.uint16))


def _masked_case(seed, B=3):
    w = dataclasses.replace(configs.MINI_V1, n_layers=2, batch=B, cross_cap=512,
                            cross_len=None, cross_len_range=(1, 512), self_len=100)
    enc = np.array([512, 300, 77][:B], np.int32)
    d = wdev.step_inputs(w, hp.DEV, cross_lens=enc, fill_lens=(np.full(B, 100),
                                                                 np.full(B, w.cross_cap)))
    rng = np.random.default_rng(seed)
    mask = rng.random((B, w.cross_cap)) < 0.4
    return w, d, enc, mask


@pytest.mark.parametrize("split", ["1", "0"])
def test_cross_mask_matches_oracle(split, tune):
    tune(attn_schedule=1 if split == "1" else 2)
    w, d, enc, mask = _masked_case(4)
    mask[2, :] = False                  # no attended key: zeros
    mask[1, 299] = True                 # the last valid key
    mask[1, 300:] = True                # bits past enc_len: ignored
    print(f"[mask] split={split} enc={enc.tolist()} attended={[int(m[:e].sum()) for m, e in zip(mask, enc)]}", flush=True)
    packed = _pack(mask)
    ws = hp.workspace(w, w.self_cap, w.cross_cap)
    o_s, o_c = hp.out_buf(w), hp.out_buf(w)
    _ex(w, d, o_s, o_c, ws, mask=_dev(packed), words=packed.shape[1])
    got = hp.host(o_c)
    q = oattn.bf16_bits_to_f64(gen.queries(w, "cross"))
    worst = 0.0
    for layer in range(w.n_layers):
        for b in range(w.batch):
            K = oattn.bf16_bits_to_f64(gen.kv_rows(w, "cross", "k", layer, b, w.cross_cap))
            V = oattn.bf16_bits_to_f64(gen.kv_rows(w, "cross", "v", layer, b, w.cross_cap))
            for h in range(w.heads):
                o = oattn.attend_masked(q[layer, b, h], K[h], V[h], enc[b], mask[b], w.scale)
                worst = max(worst, hp.row_rel_err(got[layer, b, h], o))
    assert worst <= BAR, worst
    assert not got[:, 2].any()
    # the self segment of the same launch is untouched by the mask
    s_ref, _ = hp.attn_step(w, d, ws=ws)
    assert np.array_equal(hp.host(o_s).view(np.uint32), hp.host(s_ref).view(np.uint32))


def test_all_true_mask_changes_no_bit():
    w, d, enc, mask = _masked_case(5)
    packed = _pack(np.ones_like(mask))
    ws = hp.workspace(w, w.self_cap, w.cross_cap)
    o_s, o_c = hp.out_buf(w), hp.out_buf(w)
    _ex(w, d, o_s, o_c, ws, mask=_dev(packed), words=packed.shape[1])
    r_s, r_c = hp.attn_step(w, d, ws=ws)
    assert np.array_equal(hp.host(o_c).view(np.uint32), hp.host(r_c).view(np.uint32))
    assert np.array_equal(hp.host(o_s).view(np.uint32), hp.host(r_s).view(np.uint32))


@pytest.mark.parametrize("split", ["1", "0"])
def test_fully_masked_tiles_are_not_read(split, tune):
    tune(attn_schedule=1 if split == "1" else 2)
    w, d, enc, mask = _masked_case(6)
    mask[:, 64:192] = False             # whole tiles (32-key) of every sequence
    for name in ("k_cross", "v_cross"):  # NaN there: a read of them would show
        d[name][:, :, :, 64:192, :] = float("nan")
    packed = _pack(mask)
    ws = hp.workspace(w, w.self_cap, w.cross_cap)
    o_s, o_c = hp.out_buf(w), hp.out_buf(w)
    _ex(w, d, o_s, o_c, ws, mask=_dev(packed), words=packed.shape[1])
    got = hp.host(o_c)
    assert np.all(np.isfinite(got))
    q = oattn.bf16_bits_to_f64(gen.queries(w, "cross"))
    worst = 0.0
    for layer in range(w.n_layers):
        for b in range(w.batch):
            K = oattn.bf16_bits_to_f64(gen.kv_rows(w, "cross", "k", layer, b, w.cross_cap))
            V = oattn.bf16_bits_to_f64(gen.kv_rows(w, "cross", "v", layer, b, w.cross_cap))
            for h in range(w.heads):
                o = oattn.attend_masked(q[layer, b, h], K[h], V[h], enc[b], mask[b], w.scale)
                worst = max(worst, hp.row_rel_err(got[layer, b, h], o))
    assert worst <= BAR, worst
