"""GPU parity of the pieces that make a decode step self-driving, through the C ABI:

* dec_kv_append writes the current token's rows (bit-exact against the oracle);
* dec_sample_topk_philox draws its own uniforms: the same bars as the sampler
  parity, and bit-identical outputs to dec_sample_topk given the oracle's uniforms
  (so the device generator reproduces the oracle's Philox words exactly);
* a captured step -- append, fused attention, sampling with device uniforms, advance --
  replayed several times with no host input, each replay checked against the oracle, with
  the advance as its own node or inside the sampler (dec_sample_topk_advance);
* dec_sample_topk_advance equals dec_sample_topk_ex at the counters' step bit for bit, on
  the narrow and the wide path, and leaves every counter and length one larger;
* dec_philox_uniforms draws the oracle's uniforms for a run of steps in one launch, and a
  sampler handed them samples exactly what the sampler drawing its own samples.
"""
import dataclasses

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import autoregressive_audio_token_amd as dec  # noqa: E402
from oracle import attn as oattn, cache as ocache, rng as orng  # noqa: E402
from workloads import configs, gen, device as wdev  # noqa: E402
from tests import hip_path as hp  # noqa: E402
from tests.test_gpu_sampler import _compare  # noqa: E402

BAR = 2e-3


def _dev(a, dtype=None):
    return wdev.to_device(np.asarray(a), hp.DEV, dtype)


def _bits(t):
    """Host copy of a device tensor as raw element bits (uint16 for bf16, uint32 for fp32)."""
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def d_cross_lens(w):
    """Rows drawn into the description cache: its capacity."""
    return np.full(w.batch, w.cross_cap)


def _np_bits(a):
    a = np.asarray(a)
    return a.view(np.uint16) if a.dtype == np.uint16 else a.astype(np.float32).view(np.uint32)


@pytest.mark.parametrize("base", ["mini_v1", "tiny"])
def test_append_writes_exactly_the_current_rows(base):
    w = dataclasses.replace(configs.BY_NAME[base], n_layers=2, batch=6, heads=4, self_cap=96)
    lens = [1, 96, 0, 97, 50, -3]            # first slot, last slot, none, past the end, mid, none
    print(f"[append] {w.name} dtype={w.dtype} lens={lens}", flush=True)
    k0 = gen.cache(w, "self", "k", [w.self_cap] * w.batch)
    v0 = gen.cache(w, "self", "v", [w.self_cap] * w.batch)
    kn, vn = gen.new_rows(w, "k", 0), gen.new_rows(w, "v", 0)
    kc, vc = _dev(k0), _dev(v0)
    dec.dec_kv_append(_dev(kn), _dev(vn), kc, vc, _dev(np.array(lens, np.int32)), w.n_layers,
                      w.batch, w.heads, w.self_cap, 64, hp.code(w))
    want_k, want_v = ocache.append(kn, vn, k0.copy(), v0.copy(), lens)
    assert np.array_equal(_bits(kc), _np_bits(want_k))
    assert np.array_equal(_bits(vc), _np_bits(want_v))


@pytest.mark.parametrize("name", ["tiny", "long_description", "batched_mixed"])
def test_philox_sampler_matches_oracle_and_explicit_uniforms(name):
    w = configs.BY_NAME[name]
    lg, T = gen.logits(w), gen.temperatures(w)
    steps = (np.arange(w.batch, dtype=np.int64) * 7 + 1).astype(np.int32)
    seed = 0x5EED00001234 + w.cfg_id
    print(f"[philox] {name} B={w.batch} seed={seed:#x}", flush=True)
    lg_d, T_d, st_d = _dev(lg), _dev(T), _dev(steps)
    B, k = w.batch, w.top_k
    tok = torch.full((B, 9), -7, dtype=torch.int32, device=hp.DEV)
    idx = torch.full((B, 9, k), -7, dtype=torch.int32, device=hp.DEV)
    prob = torch.full((B, 9, k), float("nan"), dtype=torch.float32, device=hp.DEV)
    dec.dec_sample_topk_philox(lg_d, B, 9, w.vocab_valid, w.vocab_stride, T_d, k, seed, st_d,
                               w.fill_token, tok, idx, prob)
    u = orng.sample_uniforms(seed, steps, 9)
    _compare(lg, w.vocab_valid, T, k, u, steps, w.fill_token, tok, idx, prob)
    t2, i2, p2 = hp.sample(w, lg_d, T_d, _dev(u), step=st_d)
    assert np.array_equal(hp.host(tok), hp.host(t2))
    assert np.array_equal(hp.host(idx), hp.host(i2))
    assert np.array_equal(_bits(prob), _bits(p2))


def test_philox_sampler_without_step_uses_step_zero_and_no_delay():
    w = configs.MINI_V1
    lg, T = gen.logits(w), gen.temperatures(w)
    seed = 424242
    tok = torch.full((1, 9), -7, dtype=torch.int32, device=hp.DEV)
    dec.dec_sample_topk_philox(_dev(lg), 1, 9, w.vocab_valid, w.vocab_stride, _dev(T), w.top_k,
                               seed, None, w.fill_token, tok)
    u = orng.sample_uniforms(seed, [0], 9)
    t2, _, _ = hp.sample(w, _dev(lg), _dev(T), _dev(u))
    assert np.array_equal(hp.host(tok), hp.host(t2))
    assert np.all(hp.host(tok) != w.fill_token)


@pytest.mark.parametrize("fused,fused_append", [(False, False), (True, False), (True, True)])
def test_self_driving_captured_step_matches_oracle(fused, fused_append):
    w = dataclasses.replace(configs.MINI_V1, n_layers=4, self_cap=512, self_len=200)
    L0, N, seed = w.self_len, 4, 77
    print(f"[selfdrive] NL={w.n_layers} L0={L0} replays={N} fused_advance={fused} "
          f"fused_append={fused_append}", flush=True)
    d = wdev.step_inputs(w, hp.DEV)
    kn, vn = gen.new_rows(w, "k", 0), gen.new_rows(w, "v", 0)
    kn_d, vn_d = _dev(kn), _dev(vn)
    len_g = torch.tensor([L0], dtype=torch.int32, device=hp.DEV)
    step_g = torch.tensor([0], dtype=torch.int32, device=hp.DEV)
    step_rows = torch.zeros((1, 9), dtype=torch.int32, device=hp.DEV)   # fused: one per row
    ws, nb = hp.workspace(w, w.self_cap, w.cross_cap)
    o_s, o_c = hp.out_buf(w), hp.out_buf(w)
    tok = torch.zeros((1, 9), dtype=torch.int32, device=hp.DEV)
    idx = torch.zeros((1, 9, w.top_k), dtype=torch.int32, device=hp.DEV)
    prob = torch.zeros((1, 9, w.top_k), dtype=torch.float32, device=hp.DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dec.dec_graph_begin(s)
        if fused_append:          # append and attention in one launch
            dec.dec_attn_step_append(d["q_self"], d["k_self"], d["v_self"], len_g, w.self_cap,
                                     o_s, kn_d, vn_d, d["q_cross"], d["k_cross"], d["v_cross"],
                                     d["enc_len"], w.cross_cap, o_c, w.n_layers, 1, w.heads, 64,
                                     dec.DEC_BF16, w.scale, ws, nb, s)
        else:
            dec.dec_kv_append(kn_d, vn_d, d["k_self"], d["v_self"], len_g, w.n_layers, 1,
                              w.heads, w.self_cap, 64, dec.DEC_BF16, s)
            dec.dec_attn_step(d["q_self"], d["k_self"], d["v_self"], len_g, w.self_cap, o_s,
                              d["q_cross"], d["k_cross"], d["v_cross"], d["enc_len"],
                              w.cross_cap, o_c, w.n_layers, 1, w.heads, 64, dec.DEC_BF16,
                              w.scale, ws, nb, s)
        if fused:
            dec.dec_sample_topk_advance(d["logits"], dec.DEC_F32, 1, 9, w.vocab_valid,
                                        w.vocab_stride, d["temperature"], w.top_k, None, seed,
                                        step_rows, len_g, w.fill_token, tok, idx, prob, s)
        else:
            dec.dec_sample_topk_philox(d["logits"], 1, 9, w.vocab_valid, w.vocab_stride,
                                       d["temperature"], w.top_k, seed, step_g, w.fill_token,
                                       tok, idx, prob, s)
            dec.dec_step_advance(len_g, step_g, 1, s)
        exe = dec.dec_graph_end(s)

    # oracle state: generator rows below L0 - 1, then the appended row at every later slot
    q = oattn.bf16_bits_to_f64(gen.queries(w, "self"))
    K = [oattn.bf16_bits_to_f64(gen.kv_rows(w, "self", "k", l, 0, L0)) for l in range(w.n_layers)]
    V = [oattn.bf16_bits_to_f64(gen.kv_rows(w, "self", "v", l, 0, L0)) for l in range(w.n_layers)]
    lg, T = gen.logits(w), gen.temperatures(w)
    try:
        for i in range(N):
            n = L0 + i
            for l in range(w.n_layers):      # the row this replay appends
                K[l] = np.concatenate([K[l][:, :n - 1], oattn.bf16_bits_to_f64(kn[l, 0])[:, None]], 1)
                V[l] = np.concatenate([V[l][:, :n - 1], oattn.bf16_bits_to_f64(vn[l, 0])[:, None]], 1)
            dec.dec_graph_launch(exe, s)
            s.synchronize()
            got = hp.host(o_s)
            want = np.stack([np.stack([oattn.attend_one(q[l, 0, h], K[l][h], V[l][h], n, w.scale)
                                       for h in range(w.heads)]) for l in range(w.n_layers)])
            err = hp.row_rel_err(got[:, 0], want)
            assert err <= BAR, f"replay {i}: self-attention rel err {err:.2e}"
            u = orng.sample_uniforms(seed, [i], 9)
            _compare(lg, w.vocab_valid, T, w.top_k, u, np.array([i], np.int32), w.fill_token,
                     tok, idx, prob)
            assert hp.host(len_g)[0] == n + 1
            if fused:
                assert np.all(hp.host(step_rows) == i + 1)
            else:
                assert hp.host(step_g)[0] == i + 1
        kc = _bits(d["k_self"])[:, 0]
        for l in range(w.n_layers):
            for j in range(L0 - 1, L0 - 1 + N):
                assert np.array_equal(kc[l, :, j], kn[l, 0]), (l, j)
    finally:
        dec.dec_graph_destroy(exe)


@pytest.mark.parametrize("k,uniforms", [(50, False), (50, True), (250, False)])
def test_advancing_sampler_equals_sampler_at_each_step(k, uniforms):
    # 12 captured replays from steps 0, 3, 8, 9, 100 (the delay mask opens codebook by
    # codebook for the first rows); each replay equals dec_sample_topk_ex at that step
    B, n_cb, V, S, seed = 5, 9, 1089, 1096, 0x0123_4567_89AB_CDEF
    rng = np.random.default_rng(7 + k)
    lg = np.full((B, n_cb, S), 1e30, np.float32)
    lg[:, :, :V] = rng.standard_normal((B, n_cb, V), dtype=np.float32) * 3
    T = np.array([1.0, 0.0, 0.7, 1.3, 1.0], np.float32)
    step0 = np.array([0, 3, 8, 9, 100], np.int32)
    len0 = np.array([10, 20, 30, 40, 50], np.int32)
    print(f"[advance] k={k} uniforms={uniforms}", flush=True)
    lg_d, T_d = _dev(lg), _dev(T)
    u_d = _dev(rng.random((B, n_cb), dtype=np.float32)) if uniforms else None
    step_rows = _dev(np.repeat(step0[:, None], n_cb, 1))
    len_d = _dev(len0)
    outs = [torch.zeros((B, n_cb), dtype=torch.int32, device=hp.DEV),
            torch.zeros((B, n_cb, k), dtype=torch.int32, device=hp.DEV),
            torch.zeros((B, n_cb, k), dtype=torch.float32, device=hp.DEV)]
    refs = [torch.empty_like(t) for t in outs]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dec.dec_graph_begin(s)
        dec.dec_sample_topk_advance(lg_d, dec.DEC_F32, B, n_cb, V, S, T_d, k, u_d, seed,
                                    step_rows, len_d, 1089, *outs, s)
        exe = dec.dec_graph_end(s)
    try:
        for i in range(12):
            dec.dec_graph_launch(exe, s)
            s.synchronize()
            dec.dec_sample_topk_ex(lg_d, dec.DEC_F32, B, n_cb, V, S, T_d, k, u_d, seed,
                                   _dev(step0 + i), 1089, *refs)
            torch.cuda.synchronize()
            for a, r in zip(outs, refs):
                assert np.array_equal(_bits(a), _bits(r)), f"replay {i}"
            assert np.array_equal(hp.host(step_rows), np.repeat(step0[:, None] + i + 1, n_cb, 1))
            assert np.array_equal(hp.host(len_d), len0 + i + 1)
    finally:
        dec.dec_graph_destroy(exe)


@pytest.mark.parametrize("split,chunk", [("0", None), ("1", None), ("1", "128"), ("1", "256")])
def test_fused_append_equals_append_then_attention(split, chunk, tune):
    # dec_attn_step_append against dec_kv_append + dec_attn_step on copies of the same
    # caches: outputs and both caches bit for bit.  Lengths at tile and chunk edges, the
    # full capacity, past it and non-positive (those append nothing).
    tune(attn_schedule=1 if split == "1" else 2)
    if chunk:
        tune(attn_chunk_keys=int(chunk))
    lens = np.array([1, 2, 32, 33, 64, 65, 129, 1024, 1025, 2048, 2049, 3000, 0, -3], np.int32)
    w = dataclasses.replace(configs.MINI_V1, n_layers=2, batch=len(lens), self_cap=2048,
                            self_len=None, self_len_range=(1, 2))
    print(f"[fused append] split={split} chunk={chunk} lens={lens.tolist()}", flush=True)
    d = wdev.step_inputs(w, hp.DEV, self_lens=lens,
                         fill_lens=(np.full(len(lens), w.self_cap), d_cross_lens(w)))
    kn, vn = _dev(gen.new_rows(w, "k", 3)), _dev(gen.new_rows(w, "v", 3))
    ws, nb = hp.workspace(w, w.self_cap, w.cross_cap)
    k2, v2 = d["k_self"].clone(), d["v_self"].clone()
    ref_s, ref_c = hp.out_buf(w), hp.out_buf(w)
    dec.dec_kv_append(kn, vn, k2, v2, d["len"], w.n_layers, w.batch, w.heads, w.self_cap, 64,
                      dec.DEC_BF16)
    dec.dec_attn_step(d["q_self"], k2, v2, d["len"], w.self_cap, ref_s, d["q_cross"],
                      d["k_cross"], d["v_cross"], d["enc_len"], w.cross_cap, ref_c, w.n_layers,
                      w.batch, w.heads, 64, dec.DEC_BF16, w.scale, ws, nb)
    o_s, o_c = hp.out_buf(w), hp.out_buf(w)
    dec.dec_attn_step_append(d["q_self"], d["k_self"], d["v_self"], d["len"], w.self_cap, o_s,
                             kn, vn, d["q_cross"], d["k_cross"], d["v_cross"], d["enc_len"],
                             w.cross_cap, o_c, w.n_layers, w.batch, w.heads, 64, dec.DEC_BF16,
                             w.scale, ws, nb)
    assert np.array_equal(_bits(o_s), _bits(ref_s))
    assert np.array_equal(_bits(o_c), _bits(ref_c))
    assert np.array_equal(_bits(d["k_self"]), _bits(k2))
    assert np.array_equal(_bits(d["v_self"]), _bits(v2))


def test_appending_records_over_growing_lengths(tune):
    # A decode loop's self lengths grow by one per step, so a short sequence's first tile
    # straddles its length every step; the appending kernel takes key len - 1 from the new
    # rows, so a record one key shorter still serves.  Steps with and without records on
    # copies of the same caches: outputs and caches bit for bit at every step, including a
    # jump past the capacity (nothing appended: the record one key shorter must not serve)
    # and a return below it.
    w = dataclasses.replace(configs.MINI_V1, n_layers=2, batch=3, self_cap=96,
                            self_len=None, self_len_range=(1, 2))
    steps = np.array([[1, 31, 93], [2, 32, 94], [3, 33, 95], [4, 34, 98], [5, 35, 99],
                      [6, 36, 96], [7, 37, 97]], np.int32)
    print(f"[append records] lens per step {steps.tolist()}", flush=True)
    d = wdev.step_inputs(w, hp.DEV, self_lens=steps[0],
                         fill_lens=(np.full(w.batch, w.self_cap), d_cross_lens(w)))
    runs = []
    for records in (True, False):
        ws, nb = hp.workspace(w, w.self_cap, w.cross_cap)
        runs.append(dict(records=records, ws=ws, nb=nb, k=d["k_self"].clone(),
                         v=d["v_self"].clone(), len=d["len"].clone()))
    for s, lens in enumerate(steps):
        kn, vn = _dev(gen.new_rows(w, "k", s)), _dev(gen.new_rows(w, "v", s))
        outs = []
        for r in runs:
            r["len"].copy_(torch.from_numpy(lens))
            o_s, o_c = hp.out_buf(w), hp.out_buf(w)
            with hp.tuning(attn_no_records=0 if r["records"] else 1):
                dec.dec_attn_step_append(d["q_self"], r["k"], r["v"], r["len"], w.self_cap, o_s,
                                         kn, vn, d["q_cross"], d["k_cross"], d["v_cross"],
                                         d["enc_len"], w.cross_cap, o_c, w.n_layers, w.batch,
                                         w.heads, 64, dec.DEC_BF16, w.scale, r["ws"], r["nb"])
            outs.append([_bits(o_s), _bits(o_c), _bits(r["k"]), _bits(r["v"])])
        for a, b in zip(*outs):
            assert np.array_equal(a, b), (s, lens.tolist())


@pytest.mark.parametrize("seed,step0,n_steps,B,n_cb",
                         [(0x0123_4567_89AB_CDEF, 0, 64, 1, 9), (5, 2040, 8, 33, 9),
                          (0xFFFF_FFFF_FFFF_FFFF, 123456, 3, 4, 2), (0, 0, 1, 1, 1)])
def test_batch_uniforms_match_oracle(seed, step0, n_steps, B, n_cb):
    # dec_philox_uniforms: every step's [B, n_cb] block equals the oracle's Philox4x64-10
    # uniforms at that step, bit for bit
    print(f"[uniforms] seed={seed:#x} step0={step0} n_steps={n_steps} B={B} n_cb={n_cb}",
          flush=True)
    out = torch.full((n_steps, B, n_cb), -1.0, dtype=torch.float32, device=hp.DEV)
    dec.dec_philox_uniforms(seed, step0, n_steps, B, n_cb, out)
    got = hp.host(out)
    for s in range(n_steps):
        want = orng.sample_uniforms(seed, np.full(B, step0 + s), n_cb)
        assert np.array_equal(got[s].view(np.uint32), want.view(np.uint32)), f"step {step0 + s}"


@pytest.mark.parametrize("k", [50, 250])
def test_sampler_reading_batch_uniforms_equals_drawing_them(k):
    # a generation that draws its uniforms ahead (dec_philox_uniforms) and hands each step
    # its block samples exactly what the sampler drawing its own (uniforms NULL) samples:
    # 12 steps from step 5, every output bit for bit
    B, n_cb, V, S, seed, st0 = 3, 9, 1089, 1096, 0x5EED_0000_0000_0004, 5
    rng = np.random.default_rng(31 + k)
    lg = np.full((B, n_cb, S), 1e30, np.float32)
    lg[:, :, :V] = rng.standard_normal((B, n_cb, V), dtype=np.float32) * 3
    lg_d, T_d = _dev(lg), _dev(np.array([1.0, 0.7, 1.3], np.float32))
    print(f"[batch uniforms] k={k}", flush=True)
    table = torch.empty((12, B, n_cb), dtype=torch.float32, device=hp.DEV)
    dec.dec_philox_uniforms(seed, st0, 12, B, n_cb, table)
    step_a = _dev(np.full((B, n_cb), st0, np.int32))
    step_b = _dev(np.full((B, n_cb), st0, np.int32))
    mk = lambda: [torch.zeros((B, n_cb), dtype=torch.int32, device=hp.DEV),
                  torch.zeros((B, n_cb, k), dtype=torch.int32, device=hp.DEV),
                  torch.zeros((B, n_cb, k), dtype=torch.float32, device=hp.DEV)]
    drawn, read = mk(), mk()
    for i in range(12):
        dec.dec_sample_topk_advance(lg_d, dec.DEC_F32, B, n_cb, V, S, T_d, k, None, seed,
                                    step_a, None, 1089, *drawn)
        dec.dec_sample_topk_advance(lg_d, dec.DEC_F32, B, n_cb, V, S, T_d, k, table[i], seed,
                                    step_b, None, 1089, *read)
        torch.cuda.synchronize()
        for a, r in zip(drawn, read):
            assert np.array_equal(_bits(a), _bits(r)), f"step {st0 + i}"
    assert np.array_equal(hp.host(step_a), hp.host(step_b))
