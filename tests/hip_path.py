"""Calls into the HIP path through the C ABI, for the GPU tests."""
import contextlib

import numpy as np
import torch

import autoregressive_audio_token_amd as dec

DEV = "cuda:0"
HD = 64


@contextlib.contextmanager
def tuning(**fields):
    """Launch-policy overrides (dec_tuning) for the calls inside the block; the previous
    overrides come back afterwards."""
    before = dec.dec_tuning_get()
    now = dict(before)
    now.update(fields)
    dec.dec_tuning_set(**now)
    try:
        yield
    finally:
        dec.dec_tuning_set(**before)


def code(w):
    return dec.DEC_BF16 if w.dtype == "bf16" else dec.DEC_F32


def workspace(w, self_cap, cross_cap, batch=None):
    B = w.batch if batch is None else batch
    nbytes = dec.dec_attn_workspace_bytes(w.n_layers, B, w.heads, w.head_dim, self_cap, cross_cap)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    dec.dec_attn_workspace_init(ws, nbytes)
    return ws, nbytes


def out_buf(w, fill=float("nan")):
    return torch.full((w.n_layers, w.batch, w.heads, w.head_dim), fill, dtype=torch.float32,
                      device=DEV)


def attn(kind, w, d, ws=None, lens=None, scale=None, cap=None, k=None, v=None):
    """One dec_attn_self / dec_attn_cross call; returns the fp32 output tensor."""
    cap = (w.self_cap if kind == "self" else w.cross_cap) if cap is None else cap
    if ws is None:
        ws = workspace(w, cap if kind == "self" else 0, cap if kind == "cross" else 0)
    lens = (d["len"] if kind == "self" else d["enc_len"]) if lens is None else lens
    k = d[f"k_{kind}"] if k is None else k
    v = d[f"v_{kind}"] if v is None else v
    out = out_buf(w)
    fn = dec.dec_attn_self if kind == "self" else dec.dec_attn_cross
    fn(d[f"q_{kind}"], k, v, lens, out, w.n_layers, w.batch, w.heads, cap, w.head_dim, code(w),
       w.scale if scale is None else scale, ws[0], ws[1])
    return out


def attn_step(w, d, ws=None, scale=None):
    if ws is None:
        ws = workspace(w, w.self_cap, w.cross_cap)
    o_s, o_c = out_buf(w), out_buf(w)
    dec.dec_attn_step(d["q_self"], d["k_self"], d["v_self"], d["len"], w.self_cap, o_s,
                      d["q_cross"], d["k_cross"], d["v_cross"], d["enc_len"], w.cross_cap, o_c,
                      w.n_layers, w.batch, w.heads, w.head_dim, code(w),
                      w.scale if scale is None else scale, ws[0], ws[1])
    return o_s, o_c


def sample(w, logits, temperature, uniforms, step=None, top_k=None, V_valid=None,
           fill=None, B=None, n_cb=None):
    B = w.batch if B is None else B
    n_cb = w.n_codebooks if n_cb is None else n_cb
    k = w.top_k if top_k is None else top_k
    V = w.vocab_valid if V_valid is None else V_valid
    stride = logits.shape[-1]
    tokens = torch.full((B, n_cb), -7, dtype=torch.int32, device=DEV)
    idx = torch.full((B, n_cb, k), -7, dtype=torch.int32, device=DEV)
    prob = torch.full((B, n_cb, k), float("nan"), dtype=torch.float32, device=DEV)
    dec.dec_sample_topk(logits, B, n_cb, V, stride, temperature, k, uniforms, step,
                        w.fill_token if fill is None else fill, tokens, idx, prob)
    return tokens, idx, prob


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def row_rel_err(got, want):
    """max over rows (the last axis) of ||got - want||_inf / ||want||_inf (rows with
    want == 0 compare absolutely)."""
    want = np.asarray(want, np.float64)
    hd = want.shape[-1]
    got = np.asarray(got, np.float64).reshape(-1, hd)
    want = want.reshape(-1, hd)
    num = np.max(np.abs(got - want), axis=1)
    den = np.max(np.abs(want), axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))
