"""GPU parity of the merged LM head and the merged embedding sum, through the C ABI.

Bars, from the arithmetic: products of bf16 values are exact in fp32, and each output
is a sum of D (LM head) or n_cb (embedding) such terms in fp32, so the error is at most
(number of roundings) x 2^-24 x sum |terms|.  The tests hold 2e-5 (LM head, at most
~260 roundings at D = 2048) and 1e-6 (embedding) times sum |terms|.  Padding rows of W
hold NaN and padding columns of the output a sentinel: any read or write of them shows.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import autoregressive_audio_token_amd as dec  # noqa: E402
from oracle import heads as oheads, attn as oattn  # noqa: E402
from workloads import configs, gen, device as wdev  # noqa: E402
from tests import hip_path as hp  # noqa: E402

SENTINEL = np.float32(-12345.5)


def _dev(a):
    return wdev.to_device(np.asarray(a), hp.DEV)


def _bf16(rng, shape, std):
    return gen.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def _check_lm_head(B, D, seed):
    n_cb, V, S = 9, configs.VOCAB_VALID, configs.VOCAB_PADDED
    rng = np.random.default_rng(seed)
    h = _bf16(rng, (B, D), 1.0)
    W = _bf16(rng, (n_cb, S, D), 1.0 / 32)
    W[:, V:, :] = gen.BF16_NAN                       # padding rows: never read
    logits = torch.full((B, n_cb, S), float(SENTINEL), dtype=torch.float32, device=hp.DEV)
    dec.dec_lm_head(_dev(h), _dev(W), logits, B, D, n_cb, V, S)
    got = hp.host(logits)
    assert np.all(got[:, :, V:] == SENTINEL), "padding columns written"
    want = oheads.lm_head(h, W, V)
    hf = oattn.bf16_bits_to_f64(h)
    Wf = oattn.bf16_bits_to_f64(W[:, :V])
    absum = np.einsum("bd,cvd->bcv", np.abs(hf), np.abs(Wf))
    err = np.abs(got[:, :, :V] - want)
    assert np.all(err <= 2e-5 * absum), float(np.max(err / absum))
    print(f"  max err / sum|terms| = {float(np.max(err / absum)):.2e}", flush=True)


@pytest.mark.parametrize("B,D", [(1, 1024), (3, 1024), (17, 512), (32, 1024), (2, 2048),
                                 (5, 768), (1, 1536), (16, 1024), (33, 1024), (64, 1536)])
@pytest.mark.parametrize("path", ["default", "gemv", "mfma"])
def test_lm_head_matches_oracle(B, D, path, tune):
    # default: the vector-ALU kernel at B <= 2, MFMA above; gemv / mfma: that kernel at
    # every B
    if path != "default":
        tune(head_kernel=1 if path == "gemv" else 2)
    print(f"[lm_head] B={B} D={D} path={path}", flush=True)
    _check_lm_head(B, D, 1000 + B * 7 + D)


@pytest.mark.parametrize("B,D", [(3, 512), (20, 768), (40, 1024), (35, 1536), (19, 2048)])
@pytest.mark.parametrize("cfg", [11, 12, 22, 42])
def test_lm_head_every_mfma_tiling(B, D, cfg, tune):
    # each row-tile x batch-tile choice of the MFMA kernel, at every model width: partial
    # batch tiles, several passes over the batch, the last row group partly past V_valid
    tune(head_mfma_cfg=int(cfg))
    print(f"[lm_head mfma] B={B} D={D} cfg={cfg}", flush=True)
    _check_lm_head(B, D, 2000 + B * 7 + D + cfg)


@pytest.mark.parametrize("B", [1, 9])
@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_lm_head_large_vocabulary(B, path, tune):
    # 50,257 rows (odd, so the last row group is partial): many row groups per codebook;
    # padding columns untouched; the same relative bar
    tune(head_kernel=1 if path == "gemv" else 2)
    n_cb, D, V = 2, 1024, 50257
    S = V + (-V) % 8
    print(f"[lm_head large V] B={B} V={V} path={path}", flush=True)
    rng = np.random.default_rng(V + B)
    h = _bf16(rng, (B, D), 1.0)
    W = _bf16(rng, (n_cb, S, D), 1.0 / 32)
    W[:, V:, :] = gen.BF16_NAN
    logits = torch.full((B, n_cb, S), float(SENTINEL), dtype=torch.float32, device=hp.DEV)
    dec.dec_lm_head(_dev(h), _dev(W), logits, B, D, n_cb, V, S)
    got = hp.host(logits)
    assert np.all(got[:, :, V:] == SENTINEL), "padding columns written"
    want = oheads.lm_head(h, W, V)
    hf = np.abs(oattn.bf16_bits_to_f64(h))
    for c in range(n_cb):
        absum = hf @ np.abs(oattn.bf16_bits_to_f64(W[c, :V])).T
        err = np.abs(got[:, c, :V] - want[:, c])
        assert np.all(err <= 2e-5 * absum), float(np.max(err / absum))


@pytest.mark.parametrize("V", [1, 15, 16, 17, 1089])
def test_lm_head_partial_row_groups_and_unaligned_output(V):
    # a last group of 16 rows that is partly past V_valid; an output pointer that is only
    # 4-byte aligned (the MFMA path's 16-byte stores are not allowed there)
    B, D, n_cb = 4, 512, 3
    S = V + (-V) % 8
    rng = np.random.default_rng(V)
    h = _bf16(rng, (B, D), 1.0)
    W = _bf16(rng, (n_cb, S, D), 1.0 / 32)
    W[:, V:, :] = gen.BF16_NAN
    want = oheads.lm_head(h, W, V)
    for offset in (0, 1):
        buf = torch.full((B * n_cb * S + 4,), float(SENTINEL), dtype=torch.float32, device=hp.DEV)
        logits = buf[offset:offset + B * n_cb * S]
        dec.dec_lm_head(_dev(h), _dev(W), logits, B, D, n_cb, V, S)
        got = hp.host(buf)[offset:offset + B * n_cb * S].reshape(B, n_cb, S)
        assert np.all(got[:, :, V:] == SENTINEL), "padding columns written"
        assert np.all(hp.host(buf)[:offset] == SENTINEL)
        assert np.all(hp.host(buf)[offset + B * n_cb * S:] == SENTINEL)
        hf = oattn.bf16_bits_to_f64(h)
        Wf = oattn.bf16_bits_to_f64(W[:, :V])
        absum = np.einsum("bd,cvd->bcv", np.abs(hf), np.abs(Wf))
        assert np.all(np.abs(got[:, :, :V] - want) <= 2e-5 * absum)


def test_lm_head_feeds_the_sampler_layout():
    # the head writes exactly the [B, 9, 1096] layout the sampler reads
    w = configs.MINI_V1
    B, D = 2, 1024
    rng = np.random.default_rng(5)
    h = _bf16(rng, (B, D), 1.0)
    W = _bf16(rng, (9, w.vocab_stride, D), 1.0 / 32)
    logits = torch.full((B, 9, w.vocab_stride), 1e30, dtype=torch.float32, device=hp.DEV)
    dec.dec_lm_head(_dev(h), _dev(W), logits, B, D, 9, w.vocab_valid, w.vocab_stride)
    T = np.ones(B, np.float32)
    u = rng.random((B, 9), dtype=np.float32)
    tok, idx, prob = hp.sample(w, logits, _dev(T), _dev(u), B=B)
    t = hp.host(tok)
    assert np.all((t >= 0) & (t < w.vocab_valid))
    lg = hp.host(logits)
    for b in range(B):
        for c in range(9):
            top = np.argsort(-lg[b, c, :w.vocab_valid], kind="stable")[:w.top_k]
            assert set(hp.host(idx)[b, c]) == set(top.tolist())


def test_embed_sum_matches_oracle():
    n_cb, V_emb, D, B = 9, configs.VOCAB_PADDED, 1024, 6
    rng = np.random.default_rng(77)
    E = _bf16(rng, (n_cb, V_emb, D), 0.5)
    toks = rng.integers(0, configs.VOCAB_VALID, (B, n_cb)).astype(np.int32)
    toks[1, :4] = configs.VOCAB_VALID                # the fill token has a row of its own
    toks[2, 3] = -1                                  # out of range: adds nothing
    toks[3, :] = V_emb                               # all out of range: zeros
    toks[4, 8] = V_emb - 1                           # last row
    x = torch.full((B, D), float("nan"), dtype=torch.float32, device=hp.DEV)
    dec.dec_embed_sum(_dev(toks), _dev(E), x, B, n_cb, V_emb, D)
    got = hp.host(x)
    want = oheads.embed(toks, E)
    Ef = oattn.bf16_bits_to_f64(E)
    absum = np.zeros((B, D))
    for b in range(B):
        for c in range(n_cb):
            if 0 <= toks[b, c] < V_emb:
                absum[b] += np.abs(Ef[c, toks[b, c]])
    assert np.all(np.abs(got - want) <= 1e-6 * absum)
    assert np.all(got[3] == 0.0)


def test_embed_sum_at_the_largest_batch():
    # B = 65535, the most the entry accepts (one workgroup row per sequence): every row
    # against the oracle, tokens drawn from -1..V_emb (out-of-range entries add nothing)
    n_cb, V_emb, D, B = 9, configs.VOCAB_PADDED, 1024, 65535
    rng = np.random.default_rng(65535)
    E = _bf16(rng, (n_cb, V_emb, D), 0.5)
    toks = rng.integers(-1, V_emb + 1, (B, n_cb)).astype(np.int32)
    print(f"[embed max B] B={B}", flush=True)
    x = torch.full((B, D), float("nan"), dtype=torch.float32, device=hp.DEV)
    dec.dec_embed_sum(_dev(toks), _dev(E), x, B, n_cb, V_emb, D)
    got = hp.host(x)
    want = oheads.embed(toks, E)
    Ef = np.abs(oattn.bf16_bits_to_f64(E))
    ok = (toks >= 0) & (toks < V_emb)
    absum = np.zeros((B, D))
    for c in range(n_cb):
        absum += Ef[c, np.clip(toks[:, c], 0, V_emb - 1)] * ok[:, c:c + 1]
    assert np.all(np.abs(got - want) <= 1e-6 * absum)
    with pytest.raises(dec.DecError):
        dec.dec_embed_sum(_dev(toks), _dev(E), x, B + 1, n_cb, V_emb, D)
