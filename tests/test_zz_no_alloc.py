"""dec_attn_step_noalloc (the workspace-free step for callers that cannot allocate)
against dec_attn_step with a caller-owned workspace, through the C ABI.

Two calls in a row on one device's library-owned array, the second smaller than
the first.  Both shapes have fewer than 512 sequences, so their launches spread
each sequence's chunks over several workgroups and use the array's arrival
counters and chunk states.  Bar: equal bit for bit to dec_attn_step (same
kernels, same layout), and within the attention bar of the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import autoregressive_audio_token_amd as dec  # noqa: E402
from workloads import configs, device as wdev  # noqa: E402
from tests import hip_path as hp  # noqa: E402
from tests.oracle_inputs import RowSource, all_rows  # noqa: E402

BAR = 2e-3
TIGHT = 1e-4

CASES = [
    # (layers, batch, self lengths, cross lengths): the second call is the smaller one
    (4, 2, [1000, 700], [300, 64]),
    (2, 1, [257], [90]),
]


def _noalloc(w, d):
    o_s, o_c = hp.out_buf(w), hp.out_buf(w)
    dec.dec_attn_step_noalloc(d["q_self"], d["k_self"], d["v_self"], d["len"], w.self_cap, o_s,
                              d["q_cross"], d["k_cross"], d["v_cross"], d["enc_len"],
                              w.cross_cap, o_c, w.n_layers, w.batch, w.heads, w.head_dim,
                              hp.code(w), w.scale)
    return o_s, o_c


def test_noalloc_matches_workspace_step_twice_shrinking():
    base = configs.MINI_V1
    for nl, b, s_len, c_len in CASES:
        w = dataclasses.replace(base, n_layers=nl, batch=b, cross_cap=512)
        print(f"[noalloc] layers={nl} batch={b} self={s_len} cross={c_len}", flush=True)
        d = wdev.step_inputs(w, hp.DEV, self_lens=s_len, cross_lens=c_len)
        n_s, n_c = _noalloc(w, d)
        r_s, r_c = hp.attn_step(w, d)
        torch.cuda.synchronize()
        assert torch.equal(n_s, r_s) and torch.equal(n_c, r_c), "differs from dec_attn_step"
        src = RowSource(w, np.asarray(s_len), np.asarray(c_len))
        rows = all_rows(w)
        for kind, out, lens in (("self", n_s, s_len), ("cross", n_c, c_len)):
            got = hp.host(out)
            g = np.stack([got[layer, bb, h] for layer, bb, h in rows])
            want = src.expected(kind, np.asarray(lens), rows)
            err = hp.row_rel_err(g, want)
            print(f"  {kind}: rows={len(rows)} max_rel_err={err:.3e}", flush=True)
            assert np.all(np.isfinite(g)) and err <= BAR and err <= TIGHT


def test_noalloc_repeats_bitwise():
    # the array keeps the last call's contents: a repeat must start from cleared counters
    w = dataclasses.replace(configs.MINI_V1, n_layers=2, batch=1, cross_cap=512)
    d = wdev.step_inputs(w, hp.DEV, self_lens=[700], cross_lens=[64])
    first = [t.clone() for t in _noalloc(w, d)]
    for _ in range(3):
        again = _noalloc(w, d)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(first, again))
