"""The C-ABI library on the CPU: it loads, exports every declared symbol, and rejects
bad arguments on the host before any HIP call (fake device addresses are safe here
because every case below fails validation first).
"""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import autoregressive_audio_token_amd as dec
from autoregressive_audio_token_amd import decstep as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decstep.h")
A = 0x10000          # a fake, 16-byte aligned "device address" (never dereferenced)
# the workspace's first-tile records: 4 waves x 16 bytes for each of up to 4096 workgroups
REC = 4096 * 4 * 16

# These cases hand fake addresses to the library; they are host-logic tests and run
# only where no GPU is visible, so a case that slipped past validation could never
# reach a device.
_no_gpu = pytest.mark.skipif(os.environ.get("DECSTEP_FAKE_PTR_TESTS") != "1" and
                             __import__("torch").cuda.is_available(),
                             reason="fake-pointer host tests run only without a GPU")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dec_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 15
    lib = ctypes.CDLL(D.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_missing_library_fails_loudly():
    env = dict(os.environ, DECSTEP_LIB="/nonexistent/libdecstep.so")
    code = "import autoregressive_audio_token_amd as d; d.dec_attn_chunk_keys()"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True)
    assert r.returncode != 0 and "not built" in r.stderr


def test_build_module_imports_without_the_library():
    env = dict(os.environ, DECSTEP_LIB="/nonexistent/libdecstep.so")
    code = "import autoregressive_audio_token_amd.build as b; print(b.LIB)"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("libdecstep.so")


def test_importing_build_from_the_package_loads_no_library():
    # the build step must not bind the library it is about to replace: a process keeps
    # the first copy it loads, so the fresh build's new entry points would be missing
    code = ("import sys; from autoregressive_audio_token_amd import build; "
            "print('autoregressive_audio_token_amd.decstep' in sys.modules, build.__name__)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == ["False", "autoregressive_audio_token_amd.build"]


def test_strerror_names_every_status():
    for code in range(8):
        assert dec.dec_strerror(code).startswith("DEC_")
    assert "unknown" in dec.dec_strerror(99)


def _attn(**kw):
    a = dict(q=A, k=A, v=A, len=A, out=A, NL=1, B=1, H=1, L=16, hd=64, dt=0, scale=0.125,
             ws=None, wsb=0)
    a.update(kw)
    return D.raw_status("dec_attn_self", a["q"], a["k"], a["v"], a["len"], a["out"], a["NL"],
                        a["B"], a["H"], a["L"], a["hd"], a["dt"], ctypes.c_float(a["scale"]),
                        a["ws"], a["wsb"], None)


@_no_gpu
def test_attention_host_validation():
    assert _attn(q=None) == D.DEC_E_NULL
    assert _attn(len=None) == D.DEC_E_NULL
    assert _attn(dt=2) == D.DEC_E_DTYPE
    for bad in (dict(NL=0), dict(B=0), dict(H=-1), dict(L=0), dict(B=1 << 20, H=1 << 11)):
        assert _attn(**bad) == D.DEC_E_SHAPE, bad
    for hd in (32, 96, 256):                     # head dims 64 and 128 are built
        assert _attn(hd=hd) == D.DEC_E_UNSUPPORTED, hd
    assert _attn(B=5000) == D.DEC_E_UNSUPPORTED
    assert _attn(L=1 << 22, hd=128, dt=1) == D.DEC_E_UNSUPPORTED   # 2 GiB per sequence
    assert _attn(q=A + 8) == D.DEC_E_ALIGN
    assert _attn(out=A + 2) == D.DEC_E_ALIGN
    # a cache longer than one chunk needs the workspace: at least the states at 1024-key
    # chunks (two 256-byte ticket regions, 4 chunk states of 68 floats rounded to 1280 B);
    # the size asked for adds the states at 128-key chunks and the first-tile records
    L = 4 * dec.dec_attn_chunk_keys()
    need = dec.dec_attn_workspace_bytes(1, 1, 1, 64, L, 0)
    assert need == 512 + 32 * 68 * 4 + REC
    assert _attn(L=L, ws=None, wsb=0) == D.DEC_E_NULL
    assert _attn(L=L, ws=A, wsb=512 + 1280 - 1) == D.DEC_E_WORKSPACE
    assert _attn(L=L, ws=A + 4, wsb=need) == D.DEC_E_ALIGN


@_no_gpu
def test_step_validation_and_workspace_sizes():
    st = D.raw_status("dec_attn_step", A, A, A, A, 4096, A, A, A, A, None, 64, A,
                      24, 1, 16, 64, 0, ctypes.c_float(0.125), A, 16, None)
    assert st == D.DEC_E_NULL
    # required: the states at 1024-key chunks, two ticket regions of 384 sequences
    # (1536 B each) and 4 self chunks of 68 floats per sequence (the cross cache fits one)
    req = 2 * 1536 + 384 * 4 * 68 * 4
    assert dec.dec_attn_workspace_bytes(24, 1, 16, 64, 4096, 1024) > req
    st = D.raw_status("dec_attn_step", A, A, A, A, 4096, A, A, A, A, A, 1024, A,
                      24, 1, 16, 64, 0, ctypes.c_float(0.125), A, req - 1, None)
    assert st == D.DEC_E_WORKSPACE
    ck = dec.dec_attn_chunk_keys()
    assert ck == 1024
    # capacities within the smallest chunk (128 keys): no chunk states and no counters,
    # only the optional first-tile records
    assert dec.dec_attn_workspace_bytes(24, 1, 16, 64, 128, 128) == REC
    assert dec.dec_attn_workspace_bytes(24, 1, 16, 64, 129, 0) > 0
    # two ticket regions of 24 sequences (256 bytes each), then the chunk states at
    # 128-key chunks: 80 chunks of the self cache and 24 of the cross cache, 68 floats each
    s = dec.dec_attn_workspace_bytes(2, 3, 4, 64, 10 * ck, 0)
    c = dec.dec_attn_workspace_bytes(2, 3, 4, 64, 0, 3 * ck)
    both = dec.dec_attn_workspace_bytes(2, 3, 4, 64, 10 * ck, 3 * ck)
    assert s == 512 + 24 * 80 * 68 * 4 + REC and c == 512 + 24 * 24 * 68 * 4 + REC
    assert both == s + c - 512 - REC
    assert dec.dec_attn_workspace_bytes(2, 3, 4, 32, 10, 10) == 0
    # head dim 128: chunk states of 4 + 128 floats
    w128 = dec.dec_attn_workspace_bytes(2, 3, 4, 128, 10 * ck, 0)
    assert w128 == 512 + 24 * 80 * 132 * 4 + REC



@_no_gpu
def test_workspace_down_to_the_1024_key_states(tune):
    # A fixed 128-key chunk that the workspace holds no states for is refused right after
    # the workspace check, so these calls show which workspaces pass that check without
    # launching anything.
    def self_call(L_cap, ws, nbytes):
        return D.raw_status("dec_attn_self", A, A, A, A, A, 2, 3, 4, L_cap, 64, 0,
                            ctypes.c_float(0.125), ws, nbytes, None)
    with pytest.raises(D.DecError):
        tune(attn_chunk_keys=3)                                   # not a power of two
    tune(attn_chunk_keys=128)
    assert self_call(1024, None, 0) == D.DEC_E_UNSUPPORTED      # one 1024-key chunk: none
    small = 512 + 24 * 4 * 68 * 4                                 # 4 chunks at 1024 keys
    assert self_call(4096, A, small - 1) == D.DEC_E_WORKSPACE
    assert self_call(4096, A, small) == D.DEC_E_UNSUPPORTED


def _samp(**kw):
    a = dict(lg=A, B=1, ncb=9, V=1089, S=1096, T=A, k=50, u=A, step=None, fill=1089, tok=A,
             idx=None, prob=None)
    a.update(kw)
    return D.raw_status("dec_sample_topk", a["lg"], a["B"], a["ncb"], a["V"], a["S"], a["T"],
                        a["k"], a["u"], a["step"], a["fill"], a["tok"], a["idx"], a["prob"],
                        None)


@_no_gpu
def test_sampler_host_validation():
    assert _samp(lg=None) == D.DEC_E_NULL
    assert _samp(u=None) == D.DEC_E_NULL
    assert _samp(tok=None) == D.DEC_E_NULL
    for bad in (dict(B=0), dict(ncb=0), dict(V=0), dict(S=1000), dict(k=0), dict(k=65)):
        assert _samp(**bad) == D.DEC_E_SHAPE, bad
    assert _samp(V=5000, S=5000) == D.DEC_E_UNSUPPORTED
    assert _samp(lg=A + 2) == D.DEC_E_ALIGN
    assert _samp(idx=A + 1) == D.DEC_E_ALIGN


def _paged(**kw):
    a = dict(q=A, k=A, v=A, tab=A, len=A, out=A, NL=24, B=1, H=16, hd=64, bs=64, nb=100, mb=64,
             dt=0, ws=A, wsb=1 << 30)
    a.update(kw)
    return D.raw_status("dec_attn_self_paged", a["q"], a["k"], a["v"], a["tab"], a["len"],
                        a["out"], a["NL"], a["B"], a["H"], a["hd"], a["bs"], a["nb"], a["mb"],
                        a["dt"], ctypes.c_float(0.125), a["ws"], a["wsb"], None)


@_no_gpu
def test_paged_attention_host_validation():
    for k in ("q", "k", "v", "tab", "len", "out"):
        assert _paged(**{k: None}) == D.DEC_E_NULL, k
    assert _paged(dt=5) == D.DEC_E_DTYPE
    for bad in (dict(nb=0), dict(mb=0), dict(bs=0), dict(NL=0), dict(B=0),
                dict(mb=1 << 20, bs=1 << 12), dict(nb=1 << 30)):
        assert _paged(**bad) == D.DEC_E_SHAPE, bad
    for bad in (dict(bs=32), dict(bs=96), dict(bs=1 << 21), dict(hd=96)):
        assert _paged(**bad) == D.DEC_E_UNSUPPORTED, bad
    assert _paged(tab=A + 2) == D.DEC_E_ALIGN
    assert _paged(k=A + 8) == D.DEC_E_ALIGN
    need = dec.dec_attn_workspace_bytes(24, 1, 16, 64, 64 * 64, 0)
    req = 2 * 1536 + 384 * 4 * 68 * 4       # the states at 1024-key chunks (4096 keys)
    assert need > req
    assert _paged(wsb=req - 1) == D.DEC_E_WORKSPACE
    assert _paged(ws=None) == D.DEC_E_NULL
    st = D.raw_status("dec_attn_step_paged", A, A, A, None, A, 64, 100, 64, A, A, A, A, A, 64, A,
                      24, 1, 16, 64, 0, ctypes.c_float(0.125), A, 1 << 30, None)
    assert st == D.DEC_E_NULL
    st = D.raw_status("dec_attn_step_paged", A, A, A, A, A, 48, 100, 64, A, A, A, A, A, 64, A,
                      24, 1, 16, 64, 0, ctypes.c_float(0.125), A, 1 << 30, None)
    assert st == D.DEC_E_UNSUPPORTED


@_no_gpu
def test_heads_host_validation():
    def head(**kw):
        a = dict(h=A, W=A, lg=A, B=1, D=1024, ncb=9, V=1089, S=1096)
        a.update(kw)
        return D.raw_status("dec_lm_head", a["h"], a["W"], a["lg"], a["B"], a["D"], a["ncb"],
                            a["V"], a["S"], None)
    for k in ("h", "W", "lg"):
        assert head(**{k: None}) == D.DEC_E_NULL, k
    for bad in (dict(B=0), dict(ncb=0), dict(V=0), dict(S=1000), dict(D=0)):
        assert head(**bad) == D.DEC_E_SHAPE, bad
    for bad in (dict(D=1000), dict(D=4096), dict(D=64)):
        assert head(**bad) == D.DEC_E_UNSUPPORTED, bad
    assert head(h=A + 8) == D.DEC_E_ALIGN and head(W=A + 4) == D.DEC_E_ALIGN
    assert head(lg=A + 2) == D.DEC_E_ALIGN

    def emb(**kw):
        a = dict(t=A, E=A, x=A, B=1, ncb=9, V=1096, D=1024)
        a.update(kw)
        return D.raw_status("dec_embed_sum", a["t"], a["E"], a["x"], a["B"], a["ncb"], a["V"],
                            a["D"], None)
    for k in ("t", "E", "x"):
        assert emb(**{k: None}) == D.DEC_E_NULL, k
    for bad in (dict(B=0), dict(B=65536), dict(ncb=0), dict(V=0), dict(D=0)):
        assert emb(**bad) == D.DEC_E_SHAPE, bad
    assert emb(D=1020) == D.DEC_E_UNSUPPORTED
    assert emb(t=A + 2) == D.DEC_E_ALIGN and emb(E=A + 8) == D.DEC_E_ALIGN
    assert emb(x=A + 4) == D.DEC_E_ALIGN


@_no_gpu
def test_attention_ex_host_validation():
    def ex(**kw):
        a = dict(mask=A, words=32, Lc=1024, out=A, od=0)
        a.update(kw)
        return D.raw_status("dec_attn_step_ex", A, A, A, A, 4096, a["out"], A, A, A, A,
                            a["mask"], a["words"], a["Lc"], a["out"], 24, 1, 16, 64, 0, a["od"],
                            ctypes.c_float(0.125), A, 1 << 30, None)
    assert ex(od=3) == D.DEC_E_DTYPE
    assert ex(words=30) == D.DEC_E_SHAPE        # fewer than 2 words per 64 keys
    assert ex(words=33) == D.DEC_E_SHAPE        # odd
    assert ex(mask=A + 4) == D.DEC_E_ALIGN      # each tile reads an aligned 64-bit pair
    assert ex(out=A + 2, od=1) == D.DEC_E_ALIGN  # fp32 outputs need 4-byte alignment
    assert ex(out=A + 1, od=0) == D.DEC_E_ALIGN  # bf16 outputs need 2-byte alignment


def _samp_rng(**kw):
    a = dict(lg=A, B=1, ncb=9, V=1089, S=1096, T=A, k=50, seed=7, step=None, fill=1089, tok=A,
             idx=None, prob=None)
    a.update(kw)
    return D.raw_status("dec_sample_topk_philox", a["lg"], a["B"], a["ncb"], a["V"], a["S"],
                        a["T"], a["k"], ctypes.c_uint64(a["seed"]), a["step"], a["fill"],
                        a["tok"], a["idx"], a["prob"], None)


@_no_gpu
def test_philox_sampler_host_validation():
    assert _samp_rng(lg=None) == D.DEC_E_NULL
    assert _samp_rng(T=None) == D.DEC_E_NULL
    assert _samp_rng(tok=None) == D.DEC_E_NULL
    for bad in (dict(B=0), dict(ncb=0), dict(V=0), dict(S=1000), dict(k=0), dict(k=65)):
        assert _samp_rng(**bad) == D.DEC_E_SHAPE, bad
    assert _samp_rng(V=5000, S=5000) == D.DEC_E_UNSUPPORTED
    assert _samp_rng(step=A + 2) == D.DEC_E_ALIGN
    assert _samp_rng(prob=A + 1) == D.DEC_E_ALIGN


def _samp_ex(**kw):
    a = dict(lg=A, dt=0, B=1, ncb=9, V=1089, S=1096, T=A, k=250, u=None, seed=7, step=None,
             fill=1089, tok=A, idx=None, prob=None)
    a.update(kw)
    return D.raw_status("dec_sample_topk_ex", a["lg"], a["dt"], a["B"], a["ncb"], a["V"], a["S"],
                        a["T"], a["k"], a["u"], ctypes.c_uint64(a["seed"]), a["step"], a["fill"],
                        a["tok"], a["idx"], a["prob"], None)


@_no_gpu
def test_widened_sampler_host_validation():
    assert _samp_ex(lg=None) == D.DEC_E_NULL
    assert _samp_ex(T=None) == D.DEC_E_NULL
    assert _samp_ex(tok=None) == D.DEC_E_NULL
    assert _samp_ex(dt=2) == D.DEC_E_DTYPE
    for bad in (dict(B=0), dict(ncb=0), dict(V=0), dict(S=1000), dict(k=0), dict(k=4097)):
        assert _samp_ex(**bad) == D.DEC_E_SHAPE, bad
    assert _samp_ex(V=5000, S=5000) == D.DEC_E_UNSUPPORTED
    assert _samp_ex(lg=A + 2, dt=1) == D.DEC_E_ALIGN      # fp32 logits: 4-byte aligned
    assert _samp_ex(lg=A + 1, dt=0) == D.DEC_E_ALIGN      # bf16 logits: 2-byte aligned
    assert _samp_ex(u=A + 2) == D.DEC_E_ALIGN
    assert _samp_ex(prob=A + 1) == D.DEC_E_ALIGN


@_no_gpu
def test_paged_widened_step_host_validation():
    def call(tab=A, od=0, mask_words=16, **kw):
        return D.raw_status("dec_attn_step_paged_ex", A, A, A, tab, A, 64, 100, 64, A, A, A, A,
                            A, A, mask_words, 1024, A, 24, 1, 16, 64, 0, od,
                            ctypes.c_float(0.125), A, 1 << 30, None)
    assert call(tab=None) == D.DEC_E_NULL
    assert call(od=5) == D.DEC_E_DTYPE
    assert call(mask_words=15) == D.DEC_E_SHAPE      # 2 words per 64 keys, an even count


@_no_gpu
def test_fused_append_host_validation():
    def call(kn=A, vn=A, **kw):
        a = dict(q=A, len=A, out=A)
        a.update(kw)
        return D.raw_status("dec_attn_step_append", a["q"], A, A, a["len"], 4096, a["out"], kn,
                            vn, A, A, A, A, 1024, A, 24, 1, 16, 64, 0, ctypes.c_float(0.125),
                            A, 1 << 30, None)
    assert call(kn=None) == D.DEC_E_NULL
    assert call(vn=None) == D.DEC_E_NULL
    assert call(kn=A + 8) == D.DEC_E_ALIGN
    assert call(len=None) == D.DEC_E_NULL          # then dec_attn_step's own checks
    assert call(q=A + 8) == D.DEC_E_ALIGN


@_no_gpu
def test_advancing_sampler_host_validation():
    def adv(step=A, len_=A, **kw):
        a = dict(lg=A, dt=1, B=1, ncb=9, V=1089, S=1096, T=A, k=50, u=None, tok=A)
        a.update(kw)
        return D.raw_status("dec_sample_topk_advance", a["lg"], a["dt"], a["B"], a["ncb"],
                            a["V"], a["S"], a["T"], a["k"], a["u"], 7, step, len_, 1089,
                            a["tok"], None, None, None)
    assert adv(step=None) == D.DEC_E_NULL            # the counters it advances are required
    assert adv(lg=None) == D.DEC_E_NULL
    assert adv(k=0) == D.DEC_E_SHAPE
    assert adv(step=A + 2) == D.DEC_E_ALIGN
    assert adv(len_=A + 2) == D.DEC_E_ALIGN


def _append(**kw):
    a = dict(kn=A, vn=A, kc=A, vc=A, len=A, NL=24, B=1, H=16, L=4096, hd=64, dt=0)
    a.update(kw)
    return D.raw_status("dec_kv_append", a["kn"], a["vn"], a["kc"], a["vc"], a["len"], a["NL"],
                        a["B"], a["H"], a["L"], a["hd"], a["dt"], None)


@_no_gpu
def test_append_host_validation():
    for k in ("kn", "vn", "kc", "vc", "len"):
        assert _append(**{k: None}) == D.DEC_E_NULL, k
    assert _append(dt=7) == D.DEC_E_DTYPE
    for bad in (dict(NL=0), dict(B=0), dict(H=0), dict(L=0), dict(hd=0)):
        assert _append(**bad) == D.DEC_E_SHAPE, bad
    assert _append(hd=4) == D.DEC_E_UNSUPPORTED          # 8-byte rows
    assert _append(hd=2, dt=1) == D.DEC_E_UNSUPPORTED
    assert _append(NL=1 << 20, H=1 << 10, L=1 << 20) == D.DEC_E_SHAPE
    for k in ("kn", "vn", "kc", "vc"):
        assert _append(**{k: A + 8}) == D.DEC_E_ALIGN, k
    assert _append(len=A + 2) == D.DEC_E_ALIGN


@_no_gpu
def test_misc_validation():
    assert D.raw_status("dec_step_advance", A, A, 0, None) == D.DEC_E_SHAPE
    assert D.raw_status("dec_step_advance", None, None, 3, None) == D.DEC_E_NULL
    assert D.raw_status("dec_graph_begin", None) == D.DEC_E_NULL
    assert D.raw_status("dec_graph_end", None, None) == D.DEC_E_NULL
    assert D.raw_status("dec_graph_launch", None, None) == D.DEC_E_NULL
    assert D.raw_status("dec_graph_destroy", None) == D.DEC_E_NULL
    assert D.raw_status("dec_attn_workspace_init", None, 0, None) == D.DEC_OK
    assert D.raw_status("dec_attn_workspace_init", None, 64, None) == D.DEC_E_NULL
    assert D.raw_status("dec_attn_workspace_init", A + 4, 64, None) == D.DEC_E_ALIGN
    # the calibration read: pointers, a positive multiple of 16 bytes, alignment
    assert D.raw_status("dec_probe_read", None, 16, A, None) == D.DEC_E_NULL
    assert D.raw_status("dec_probe_read", A, 16, None, None) == D.DEC_E_NULL
    assert D.raw_status("dec_probe_read", A, 0, A, None) == D.DEC_E_SHAPE
    assert D.raw_status("dec_probe_read", A, 24, A, None) == D.DEC_E_SHAPE
    assert D.raw_status("dec_probe_read", A + 4, 16, A, None) == D.DEC_E_ALIGN
    assert D.raw_status("dec_probe_read", A, 16, A + 2, None) == D.DEC_E_ALIGN
    # batch uniforms: a buffer, positive counts, a non-negative first step, 31-bit totals
    U = "dec_philox_uniforms"
    assert D.raw_status(U, 7, 0, 4, 1, 9, None, None) == D.DEC_E_NULL
    for bad in ((7, -1, 4, 1, 9), (7, 0, 0, 1, 9), (7, 0, 4, 0, 9), (7, 0, 4, 1, 0),
                (7, 0x7FFFFFF0, 100, 1, 9), (7, 0, 1 << 20, 1 << 10, 9)):
        assert D.raw_status(U, *bad, A, None) == D.DEC_E_SHAPE, bad
    assert D.raw_status(U, 7, 0, 4, 1, 9, A + 2, None) == D.DEC_E_ALIGN


def test_tuning_overrides_round_trip_refuse_out_of_range_and_reset():
    before = dec.dec_tuning_get()
    try:
        dec.dec_tuning_set()
        assert all(v == 0 for v in dec.dec_tuning_get().values())
        good = dict(attn_chunk_keys=256, attn_schedule=2, attn_blocks=77, attn_no_halves=1,
                    attn_no_records=1, head_kernel=2, head_mfma_cfg=22)
        dec.dec_tuning_set(**good)
        assert dec.dec_tuning_get() == good
        bad = ([dict(attn_chunk_keys=c) for c in (-128, 64, 100, 384, 2048)] +
               [dict(attn_schedule=v) for v in (-1, 3)] + [dict(attn_blocks=-1)] +
               [dict(attn_no_halves=v) for v in (-1, 2)] +
               [dict(attn_no_records=v) for v in (-1, 2)] +
               [dict(head_kernel=v) for v in (-1, 3)] +
               [dict(head_mfma_cfg=v) for v in (-1, 1, 13, 21, 33, 41, 44, 99, 100)])
        for fields in bad:
            with pytest.raises(D.DecError) as err:
                dec.dec_tuning_set(**fields)
            assert err.value.status == D.DEC_E_SHAPE, fields
            assert dec.dec_tuning_get() == good, fields  # a refused call changes nothing
        for c in (11, 12, 22, 42):  # every instantiated tiling of the MFMA head
            dec.dec_tuning_set(head_mfma_cfg=c)
            assert dec.dec_tuning_get()["head_mfma_cfg"] == c
        for c in (128, 512, 1024):
            dec.dec_tuning_set(attn_chunk_keys=c)
            assert dec.dec_tuning_get()["attn_chunk_keys"] == c
        with pytest.raises(TypeError):
            dec.dec_tuning_set(no_such_field=1)
        dec.dec_tuning_set()
        assert all(v == 0 for v in dec.dec_tuning_get().values())
        assert D.raw_status("dec_tuning_get", None) == D.DEC_E_NULL
    finally:
        dec.dec_tuning_set(**before)


def test_tuning_overrides_belong_to_the_calling_thread():
    import threading
    before = dec.dec_tuning_get()
    seen = {}

    def other():
        seen["start"] = dec.dec_tuning_get()
        dec.dec_tuning_set(attn_blocks=5)
        seen["after"] = dec.dec_tuning_get()

    try:
        dec.dec_tuning_set(attn_schedule=1, head_kernel=1)
        t = threading.Thread(target=other)
        t.start()
        t.join()
        assert all(v == 0 for v in seen["start"].values())  # a new thread starts at defaults
        assert seen["after"]["attn_blocks"] == 5
        mine = dec.dec_tuning_get()  # the other thread's setting never reaches this one
        assert (mine["attn_schedule"], mine["head_kernel"], mine["attn_blocks"]) == (1, 1, 0)
    finally:
        dec.dec_tuning_set(**before)


def test_order_key_map_is_monotone_over_all_float32_bit_patterns():
    # Every float32 bit pattern, in increasing order of value: -inf .. -0 then +0 .. +inf.
    # Keys must increase strictly, except that -0 and +0 share a key; NaNs map outside
    # [key(-inf), key(+inf)] by sign.
    chunk = 1 << 25
    prev = None
    keys = np.empty(chunk, np.uint32)
    # negative values: bit patterns 0xFF800000 down to 0x80000000
    for hi in range(0xFF800000 + 1, 0x80000000, -chunk):
        lo = max(hi - chunk, 0x80000000)
        bits = np.arange(hi - 1, lo - 1, -1, dtype=np.int64).astype(np.uint32)
        x = bits.view(np.float32)
        k = keys[:x.size]
        dec.dec_order_keys_host(x, k, x.size)
        assert np.all(np.diff(k.astype(np.int64)) > 0)
        if prev is not None:
            assert int(k[0]) > prev
        prev = int(k[-1])
    kneg0 = prev
    for lo in range(0, 0x7F800000 + 1, chunk):
        hi = min(lo + chunk, 0x7F800000 + 1)
        bits = np.arange(lo, hi, dtype=np.int64).astype(np.uint32)
        x = bits.view(np.float32)
        k = keys[:x.size]
        dec.dec_order_keys_host(x, k, x.size)
        assert np.all(np.diff(k.astype(np.int64)) > 0)
        if lo == 0:
            assert int(k[0]) == kneg0          # -0 and +0 tie
        else:
            assert int(k[0]) > prev
        prev = int(k[-1])
    kinf = prev
    nan = np.array([0x7FC00000, 0x7F800001, 0xFFC00000, 0xFF800001], np.uint32).view(np.float32)
    kn = np.zeros(4, np.uint32)
    dec.dec_order_keys_host(nan, kn, 4)
    x = np.array([-np.inf], np.float32)
    kmin = np.zeros(1, np.uint32)
    dec.dec_order_keys_host(x, kmin, 1)
    assert kn[0] > kinf and kn[1] > kinf and kn[2] < kmin[0] and kn[3] < kmin[0]


@_no_gpu
def test_noalloc_step_host_validation():
    def call(NL=24, B=1, H=16, hd=64, dt=0, caps=(4096, 1024), q=A, **kw):
        return D.raw_status("dec_attn_step_noalloc", q, A, A, A, caps[0], A, A, A, A, A, caps[1],
                            A, NL, B, H, hd, dt, ctypes.c_float(0.125), None)
    assert call(q=None) == D.DEC_E_NULL
    assert call(dt=5) == D.DEC_E_DTYPE
    assert call(hd=96) == D.DEC_E_UNSUPPORTED
    assert call(NL=0) == D.DEC_E_SHAPE
    assert call(caps=(0, 1024)) == D.DEC_E_SHAPE
    # chunk states beyond the library's fixed array: rejected before anything is enqueued
    big = D.dec_attn_workspace_bytes(24, 64, 16, 64, 4096, 4096)
    assert big > 16 << 20
    assert call(B=64, caps=(4096, 4096)) == D.DEC_E_WORKSPACE


# ---- the Python binding's checks -------------------------------------------------------

def _prototypes():
    """{name: [(param name, is_pointer)]} from the header's function declarations."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, params in re.findall(r"\b(dec_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text):
        if params.strip() in ("", "void"):
            out[name] = []
            continue
        out[name] = [(re.findall(r"\w+", p)[-1], "*" in p or "dec_stream_t" in p)
                     for p in params.split(",")]
    return out


def test_binding_declarations_follow_the_header():
    """Every entry point the binding declares has the header's parameters: the same
    names in the same order, pointers where the header has pointers."""
    protos = _prototypes()
    for name, params in D._DECL.items():
        want = protos[name]
        got = [(p.name, p.dims is not None or p.kind == "stream") for p in params]
        # the executable graph handle is a pointer the binding takes as an integer
        want = [("exec_handle", True) if n == "exec" else (n, ptr) for n, ptr in want]
        got = [(n, True) if n == "exec_handle" else (n, ptr) for n, ptr in got]
        assert got == want, name


_SIZES = dict(n_layers=2, B=3, H=2, L_cap=5, hd=64, L_cap_self=7, L_cap_cross=6, n_cb=4,
              V_valid=40, V_stride=48, top_k=3, mask_words=2, n_blocks=3, block_size=64,
              max_blocks=2, D=16, V_emb=9, bytes=64, ws_bytes=256, n_steps=3)


def _good_call(params):
    """CPU tensors and integers that satisfy every declaration of one entry point."""
    import torch
    dt = {"x": torch.bfloat16, "o": torch.float32, "l": torch.bfloat16, "bf16": torch.bfloat16,
          "f32": torch.float32, "i32": torch.int32, "u32": torch.int32, "i64": torch.int64,
          "bytes": torch.uint8}
    ints = {n: v for n, v in _SIZES.items()}
    ints.update(dtype=D.DEC_BF16, out_dtype=D.DEC_F32, logits_dtype=D.DEC_BF16)
    args = {}
    for p in params:
        if p.dims is not None:
            shape = [d if isinstance(d, int) else ints[d] for d in p.dims]
            args[p.name] = torch.zeros(shape, dtype=dt[p.kind])
        elif p.kind == "stream":
            args[p.name] = None
        elif p.kind == "float":
            args[p.name] = 0.125
        else:
            args[p.name] = ints.get(p.name, 0)
    return args


def test_binding_rejects_bad_tensors_before_the_call():
    """For every buffer of every entry point: a wrong element type, a transposed
    (non-contiguous) view, a wrong element count, a host tensor and a numpy array are
    each refused by the binding (DecError with its status), never passed on.  Host
    tensors of the right kind are refused as not on a GPU, so nothing reaches the
    library here."""
    import torch
    for name, params in D._DECL.items():
        fn = getattr(dec, name)
        good = _good_call(params)
        buffers = [p for p in params if p.dims is not None]
        if not buffers:
            continue
        with pytest.raises(dec.DecError) as e:
            fn(**good)
        assert e.value.status == D.DEC_E_UNSUPPORTED and "not on a GPU" in str(e.value), name
        for p in buffers:
            t = good[p.name]
            bad = {}
            if p.kind != "bytes":
                other = torch.float64 if t.dtype != torch.float64 else torch.float32
                bad["dtype"] = (t.to(other), D.DEC_E_DTYPE)
                bad["count"] = (torch.cat([t.reshape(-1), t.reshape(-1)[:1]]), D.DEC_E_SHAPE)
            else:
                bad["count"] = (t[:-1], D.DEC_E_SHAPE)
            flat = t.reshape(-1)
            if flat.numel() > 1:
                wide = torch.zeros(flat.numel() * 2, dtype=t.dtype)
                bad["layout"] = (wide[::2], D.DEC_E_SHAPE)
                if t.dim() >= 2 and t.shape[-1] > 1 and t.shape[-2] > 1:
                    bad["transposed"] = (t.transpose(-1, -2), D.DEC_E_SHAPE)
            bad["numpy"] = (np.zeros(t.numel(), np.float32), D.DEC_E_UNSUPPORTED)
            for what, (value, status) in bad.items():
                args = dict(good)
                args[p.name] = value
                with pytest.raises(dec.DecError) as e:
                    fn(**args)
                assert e.value.status == status, (name, p.name, what, str(e.value))
                assert p.name in str(e.value), (name, p.name, what, str(e.value))


@_no_gpu
def test_binding_passes_raw_addresses_and_none_unchecked():
    """Integers are device addresses and None is NULL: the binding leaves them to the
    library, whose own check answers (here DEC_E_NULL for a required NULL)."""
    with pytest.raises(dec.DecError) as e:
        dec.dec_step_advance(None, None, 3, None)
    assert e.value.status == D.DEC_E_NULL
    with pytest.raises(dec.DecError) as e:
        dec.dec_probe_read(None, 16, A, None)
    assert e.value.status == D.DEC_E_NULL


def test_host_key_map_checks_its_arrays():
    x = np.zeros(4, np.float32)
    with pytest.raises(dec.DecError):
        dec.dec_order_keys_host(x, np.zeros(4, np.int32), 4)
    with pytest.raises(dec.DecError):
        dec.dec_order_keys_host(x, np.zeros(3, np.uint32), 4)
    with pytest.raises(dec.DecError):
        dec.dec_order_keys_host(x.astype(np.float64), np.zeros(4, np.uint32), 4)
