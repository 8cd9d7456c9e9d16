"""A whole decode step captured as one hipGraph and replayed (GPU, through the C ABI).

Each replay runs the fused self+cross attention over all layers, the sampler
with the delay mask, and the on-device len/step advance.  Every replay is
checked bit for bit against the same calls made eagerly at the matching
length, with eager work and synchronisations between replays.  A second graph
chains the widened entry points: embedding sum, the MFMA LM head feeding the
wide sampler (device-drawn uniforms), masked head-dim-128 attention with bf16
outputs, and the advance.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import autoregressive_audio_token_amd as dec  # noqa: E402
from workloads import configs, gen, device as wdev  # noqa: E402
from tests import hip_path as hp  # noqa: E402


def test_captured_step_replays_match_eager():
    w = configs.LONG_OUTPUT
    L0 = 1000
    fill = (np.full(w.batch, 1100), np.full(w.batch, w.cross_len))
    print(f"[graph] workload={w.name} L0={L0}", flush=True)
    d = wdev.step_inputs(w, hp.DEV, self_lens=[L0], fill_lens=fill)
    s = torch.cuda.Stream()
    nbytes = dec.dec_attn_workspace_bytes(w.n_layers, w.batch, w.heads, 64, w.self_cap,
                                          w.cross_cap)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=hp.DEV)
    len_g = torch.tensor([L0], dtype=torch.int32, device=hp.DEV)
    step_g = torch.tensor([0], dtype=torch.int32, device=hp.DEV)
    o_s, o_c = hp.out_buf(w), hp.out_buf(w)
    tok = torch.zeros((1, 9), dtype=torch.int32, device=hp.DEV)
    idx = torch.zeros((1, 9, 50), dtype=torch.int32, device=hp.DEV)
    prob = torch.zeros((1, 9, 50), dtype=torch.float32, device=hp.DEV)

    def step_calls(len_t, step_t, outs, stream):
        dec.dec_attn_step(d["q_self"], d["k_self"], d["v_self"], len_t, w.self_cap, outs[0],
                          d["q_cross"], d["k_cross"], d["v_cross"], d["enc_len"], w.cross_cap,
                          outs[1], w.n_layers, 1, w.heads, 64, dec.DEC_BF16, w.scale, ws, nbytes,
                          stream)
        dec.dec_sample_topk(d["logits"], 1, 9, w.vocab_valid, w.vocab_stride, d["temperature"],
                            50, d["uniforms"], step_t, w.fill_token, outs[2], outs[3], outs[4],
                            stream)

    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dec.dec_attn_workspace_init(ws, nbytes, s)
        s.synchronize()
        dec.dec_graph_begin(s)
        step_calls(len_g, step_g, (o_s, o_c, tok, idx, prob), s)
        dec.dec_step_advance(len_g, step_g, 1, s)
        exe = dec.dec_graph_end(s)
    try:
        for i in range(6):
            dec.dec_graph_launch(exe, s)
            s.synchronize()
            got = [hp.host(t) for t in (o_s, o_c, tok, idx, prob)]
            # eager reference at the same length and step, with fresh outputs
            e_len = torch.tensor([L0 + i], dtype=torch.int32, device=hp.DEV)
            e_step = torch.tensor([i], dtype=torch.int32, device=hp.DEV)
            eo = (hp.out_buf(w), hp.out_buf(w), torch.zeros_like(tok), torch.zeros_like(idx),
                  torch.zeros_like(prob))
            with torch.cuda.stream(s):
                step_calls(e_len, e_step, eo, s)
            s.synchronize()
            want = [hp.host(t) for t in eo]
            for g, e in zip(got, want):
                assert np.array_equal(g, e), f"replay {i} differs from eager"
            toks = got[2][0]
            assert all((toks[c] == w.fill_token) == (i < c) for c in range(9))
            assert hp.host(len_g)[0] == L0 + i + 1 and hp.host(step_g)[0] == i + 1
    finally:
        dec.dec_graph_destroy(exe)


def test_captured_widened_step_replays_match_eager():
    # embedding sum -> (decoder elided) -> MFMA LM head -> wide sampler with device-drawn
    # uniforms, plus masked head-dim-128 attention with bf16 outputs and the advance
    import dataclasses
    w = dataclasses.replace(configs.MINI_V1, n_layers=2, batch=4, heads=8, head_dim=128,
                            scale=128 ** -0.5, qkv_std=128 ** -0.5, self_cap=2048, cross_cap=256,
                            cross_len=None, cross_len_range=(0, 256))
    B, D, V, S, k = w.batch, 1024, w.vocab_valid, w.vocab_stride, 250
    L0 = np.array([300, 1025, 1, 2000], np.int32)
    enc = np.array([256, 100, 17, 0], np.int32)
    print(f"[graph ex] B={B} hd=128 lens={L0.tolist()} enc={enc.tolist()} k={k}", flush=True)
    d = wdev.step_inputs(w, hp.DEV, self_lens=L0, cross_lens=enc,
                         fill_lens=(np.full(B, 2048), enc))
    rng = np.random.default_rng(77)
    mask = rng.random((B, w.cross_cap)) < 0.5
    words = 2 * ((w.cross_cap + 63) // 64)
    packed = np.zeros((B, words), np.uint32)
    for j in range(w.cross_cap):
        packed[:, j // 32] |= mask[:, j].astype(np.uint32) << np.uint32(j % 32)
    mask_d = wdev.to_device(packed, hp.DEV)
    bf = lambda shape, std: wdev.to_device(gen.f32_to_bf16_bits(
        rng.standard_normal(shape, dtype=np.float32) * np.float32(std)), hp.DEV)
    h, W, E = bf((B, D), 1.0), bf((9, S, D), 1 / 32), bf((9, S, D), 0.5)
    seed = 0xC0FFEE
    nbytes = dec.dec_attn_workspace_bytes(w.n_layers, B, w.heads, 128, w.self_cap, w.cross_cap)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=hp.DEV)
    s = torch.cuda.Stream()
    len_g = torch.from_numpy(L0.copy()).to(hp.DEV)
    step_g = torch.zeros(B, dtype=torch.int32, device=hp.DEV)

    def bufs():
        shape = (w.n_layers, B, w.heads, 128)
        return dict(x=torch.zeros((B, D), dtype=torch.float32, device=hp.DEV),
                    logits=torch.zeros((B, 9, S), dtype=torch.float32, device=hp.DEV),
                    o_s=torch.zeros(shape, dtype=torch.bfloat16, device=hp.DEV),
                    o_c=torch.zeros(shape, dtype=torch.bfloat16, device=hp.DEV),
                    tok=torch.zeros((B, 9), dtype=torch.int32, device=hp.DEV),
                    idx=torch.zeros((B, 9, k), dtype=torch.int32, device=hp.DEV),
                    prob=torch.zeros((B, 9, k), dtype=torch.float32, device=hp.DEV))

    def calls(tok_in, len_t, step_t, o, stream):
        dec.dec_embed_sum(tok_in, E, o["x"], B, 9, S, D, stream)
        dec.dec_lm_head(h, W, o["logits"], B, D, 9, V, S, stream)
        dec.dec_attn_step_ex(d["q_self"], d["k_self"], d["v_self"], len_t, w.self_cap, o["o_s"],
                             d["q_cross"], d["k_cross"], d["v_cross"], d["enc_len"], mask_d, words,
                             w.cross_cap, o["o_c"], w.n_layers, B, w.heads, 128, dec.DEC_BF16,
                             dec.DEC_BF16, w.scale, ws, nbytes, stream)
        dec.dec_sample_topk_ex(o["logits"], dec.DEC_F32, B, 9, V, S, d["temperature"], k, None,
                               seed, step_t, w.fill_token, o["tok"], o["idx"], o["prob"], stream)

    g = bufs()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dec.dec_attn_workspace_init(ws, nbytes, s)
        s.synchronize()
        dec.dec_graph_begin(s)
        calls(g["tok"], len_g, step_g, g, s)
        dec.dec_step_advance(len_g, step_g, B, s)
        exe = dec.dec_graph_end(s)
    try:
        for i in range(5):
            tok_prev = g["tok"].clone()          # eager work between replays
            s.wait_stream(torch.cuda.current_stream())
            dec.dec_graph_launch(exe, s)
            s.synchronize()
            bits = lambda t: hp.host(t.view(torch.int16) if t.dtype == torch.bfloat16 else t)
            got = {kname: bits(t) for kname, t in g.items()}
            e = bufs()
            e_len = torch.from_numpy(L0 + i).to(hp.DEV)
            e_step = torch.full((B,), i, dtype=torch.int32, device=hp.DEV)
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                calls(tok_prev, e_len, e_step, e, s)
            s.synchronize()
            for kname, t in e.items():
                assert np.array_equal(got[kname].view(np.uint8), bits(t).view(np.uint8)), \
                    f"replay {i}: {kname} differs from eager"
            assert np.array_equal(hp.host(len_g), L0 + i + 1)
            assert np.all(hp.host(step_g) == i + 1)
    finally:
        dec.dec_graph_destroy(exe)
