"""A whole decode step captured as one hipGraph and replayed (GPU, through the C ABI).

Each replay runs the fused self+cross attention over all layers, the sampler
with the delay mask, and the on-device len/step advance.  Every replay is
checked bit for bit against the same calls made eagerly at the matching
length, with eager work and synchronisations between replays.
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
