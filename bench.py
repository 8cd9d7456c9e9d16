#!/usr/bin/env python3
"""Decode-step benchmark of the hot path on one MI355X.

A step is one pass of the whole hot path over one batch: self-attention over
the valid prefix of the static cache and cross-attention over the description
for all layers (one fused launch), then the fused top-k sampler over the 9
codebooks.  Exactly --warmup untimed and --steps timed steps run, each on the
next of R cache sets in rotation; the sets are distinct allocations, so each
step reads cold data (R x valid bytes exceeds the 256 MB Infinity Cache).  The
timed steps run as one captured hipGraph timed with HIP events; clock-reading
nodes inside it split them into min(10, steps) blocks (per-block step times
beside the total).

Prints ONE JSON line: value = valid K/V bytes per step / time per step (GB/s).

    python bench.py [--steps K] [--warmup W] [--workload long_description]
"""
import argparse
import dataclasses
import json
import math
import os
import platform
import statistics
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
METRIC = "decode-step µs and achieved HBM GB/s (valid KV bytes) vs MI355X peak"


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="long_description")
    ap.add_argument("--sets", type=int, default=0, help="cache sets (0: enough for >= 1 GiB)")
    ap.add_argument("--kernel-launches", type=int, default=200,
                    help="event-timed attention launches for the roofline leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--paged", type=int, default=0, metavar="BS",
                    help="self-attention cache as a paged block pool with BS keys per block\n"
                         "(blocks scattered by a seeded permutation); 0: the static cache")
    ap.add_argument("--heads", action="store_true",
                    help="time the merged LM head (and the merged embedding sum) of the\n"
                         "workload's batch instead of the attention + sampling step")
    ap.add_argument("--d-model", type=int, default=0, choices=(0, 512, 768, 1024, 1536, 2048),
                    help="with --heads: the model width (0: the workload's, 1024)")
    ap.add_argument("--batch", type=int, default=0,
                    help="with --heads: the batch size (0: the workload's)")
    ap.add_argument("--eager", action="store_true",
                    help="run warmup + steps eager steps (no graph, no timing) and exit;\n"
                         "the launch sequence the hardware-counter runs profile")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run a plain device copy of this many MiB five times and exit;\n"
                         "the calibration for the HBM byte counters")
    ap.add_argument("--head-dim", type=int, default=64, choices=(64, 128),
                    help="128: the same model width as heads of 128 (half the heads)")
    ap.add_argument("--cross-mask", type=float, default=0.0, metavar="P",
                    help="a boolean description mask keeping each key with probability P\n"
                         "(seeded), through the widened entry dec_attn_step_ex")
    ap.add_argument("--mask-runs", type=int, default=0, metavar="R",
                    help="with --cross-mask: masked keys come in runs of R keys (0: single keys)")
    ap.add_argument("--out-bf16", action="store_true",
                    help="bf16 attention outputs, through dec_attn_step_ex")
    ap.add_argument("--top-k", type=int, default=0,
                    help="sampler top_k (0: the workload's); above 64 through dec_sample_topk_ex")
    ap.add_argument("--logits-bf16", action="store_true",
                    help="bf16 logits, through dec_sample_topk_ex")
    ap.add_argument("--schedule", default="stacked", choices=("stacked", "model"),
                    help="stacked: one attention launch for all layers (self + cross);\n"
                         "model: per-layer launches, 24 x (self, cross) + the sampler per step")
    ap.add_argument("--decode-loop", action="store_true",
                    help="a workload with a step count (long_output): the whole generation,\n"
                         "lengths and steps advanced on the device, timed end to end")
    ap.add_argument("--draw-in-sampler", action="store_true",
                    help="with --decode-loop: each sampler launch draws its own uniforms "
                         "(Philox in the launch) instead of reading them from one "
                         "dec_philox_uniforms launch at the start of the generation")
    ap.add_argument("--separate-append", action="store_true",
                    help="with --decode-loop: append the current token's rows with\n"
                         "dec_kv_append as a node of its own (for comparison)")
    ap.add_argument("--attn-chunk", type=int, default=0, metavar="KEYS",
                    help="keys per split-K chunk of every attention launch (a power of two,\n"
                         "128-1024; 0: the launcher chooses), through dec_tuning_set")
    ap.add_argument("--calibrate", action="store_true",
                    help="the calibration kernels: streaming reads at 4 MiB, the workload's\n"
                         "valid bytes and 4 GiB, and the cost of an empty graph node")
    a = ap.parse_args(argv)
    if a.steps < 1 or a.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    if a.attn_chunk and (a.attn_chunk < 128 or a.attn_chunk > 1024 or
                         a.attn_chunk & (a.attn_chunk - 1)):
        ap.error("--attn-chunk must be a power of two from 128 to 1024")
    return a


def read_probe(dec, torch, nbytes, dev, stream, launches, min_pool=1 << 30):
    """Average launch time (us) of dec_probe_read over nbytes, as a captured graph of
    `launches` back-to-back launches over rotating buffers (together at least min_pool
    bytes, so with min_pool above the 256 MB Infinity Cache every launch reads HBM);
    returns (us, GB/s, buffers)."""
    sets = max(1, math.ceil(min_pool / nbytes)) if min_pool else 1
    pool = torch.zeros(sets * nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    bufs = [pool[i * nbytes:(i + 1) * nbytes] for i in range(sets)]
    n = max(launches, sets)
    with torch.cuda.stream(stream):
        for b in bufs:
            dec.dec_probe_read(b, nbytes, sink, stream)
        dec.dec_graph_begin(stream)
        for i in range(n):
            dec.dec_probe_read(bufs[i % sets], nbytes, sink, stream)
        g = dec.dec_graph_end(stream)
        dec.dec_graph_launch(g, stream)
    stream.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record(stream)
    for _ in range(reps):
        dec.dec_graph_launch(g, stream)
    e1.record(stream)
    stream.synchronize()
    dec.dec_graph_destroy(g)
    us = e0.elapsed_time(e1) * 1e3 / (reps * n)
    del pool, bufs
    return us, nbytes / (us * 1e-6) / 1e9, sets


def decode_loop(a):
    """The whole generation of a workload with a step count: step s appends the current
    token's key and value rows and attends over s + 1 self keys (and the description) in
    one launch, then samples with Philox uniforms drawn from (seed, step) and the delay mask
    and advances the lengths and steps in the sampler's own launch: two graph nodes per
    step.  The whole generation is one captured graph, its steps on R cache sets in turn,
    timed end to end."""
    import numpy as np
    import torch
    import autoregressive_audio_token_amd as dec
    from workloads import configs, gen, device as wdev

    w = configs.BY_NAME[a.workload]
    if w.n_steps <= 1:
        print(f"--decode-loop needs a workload of several steps; {w.name} is one step",
              file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)
    S = w.n_steps
    B = w.batch
    c_len = np.full(B, w.cross_len, np.int32)
    # every row a step can reach is drawn: the self cache up to the last step's length
    fill = (np.full(B, min(S, w.self_cap)), c_len)
    log(f"workload {w.name}: staging inputs for {S} steps")
    d = wdev.step_inputs(w, dev, self_lens=np.ones(B, np.int32), cross_lens=c_len,
                         fill_lens=fill)
    R = a.sets if a.sets > 0 else 8
    big = ("k_self", "v_self", "k_cross", "v_cross")
    sets = [{k: d[k] for k in big}]
    for _ in range(R - 1):
        sets.append({k: torch.empty_like(d[k]).copy_(d[k]) for k in big})
    code = dec.DEC_BF16 if w.dtype == "bf16" else dec.DEC_F32
    nb = dec.dec_attn_workspace_bytes(w.n_layers, B, w.heads, w.head_dim, w.self_cap,
                                      w.cross_cap)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    o_s = torch.empty((w.n_layers, B, w.heads, w.head_dim), dtype=torch.float32, device=dev)
    o_c = torch.empty_like(o_s)
    tok = torch.empty((B, w.n_codebooks), dtype=torch.int32, device=dev)
    k_new = wdev.to_device(gen.new_rows(w, "k", 0), dev)      # the current token's rows
    v_new = wdev.to_device(gen.new_rows(w, "v", 0), dev)
    len_d = d["len"]
    step_d = torch.zeros((B, w.n_codebooks), dtype=torch.int32, device=dev)  # one per row
    seed = 0x5EED_0000_0000_0004
    # the generation's uniforms, drawn in one launch at its start: step s reads block s
    # (the same values the sampler would draw at step s)
    table = torch.empty((S, B, w.n_codebooks), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)

    def step(st, s, i):
        if a.separate_append:
            dec.dec_kv_append(k_new, v_new, st["k_self"], st["v_self"], len_d, w.n_layers, B,
                              w.heads, w.self_cap, w.head_dim, code, s)
            dec.dec_attn_step(d["q_self"], st["k_self"], st["v_self"], len_d, w.self_cap, o_s,
                              d["q_cross"], st["k_cross"], st["v_cross"], d["enc_len"],
                              w.cross_cap, o_c, w.n_layers, B, w.heads, w.head_dim, code,
                              w.scale, ws, nb, s)
        else:
            dec.dec_attn_step_append(d["q_self"], st["k_self"], st["v_self"], len_d,
                                     w.self_cap, o_s, k_new, v_new, d["q_cross"],
                                     st["k_cross"], st["v_cross"], d["enc_len"], w.cross_cap,
                                     o_c, w.n_layers, B, w.heads, w.head_dim, code, w.scale,
                                     ws, nb, s)
        dec.dec_sample_topk_advance(d["logits"], dec.DEC_F32, B, w.n_codebooks, w.vocab_valid,
                                    w.vocab_stride, d["temperature"], w.top_k,
                                    None if a.draw_in_sampler else table[i], seed,
                                    step_d, len_d, w.fill_token, tok, None, None, s)

    def reset():
        len_d.fill_(1)
        step_d.fill_(0)

    with torch.cuda.stream(stream):
        dec.dec_attn_workspace_init(ws, nb, stream)
        dec.dec_graph_begin(stream)             # the whole generation as one graph
        if not a.draw_in_sampler:
            dec.dec_philox_uniforms(seed, 0, S, B, w.n_codebooks, table, stream)
        for s in range(S):
            step(sets[s % R], stream, s)
        graph = dec.dec_graph_end(stream)
        reset()
        dec.dec_graph_launch(graph, stream)     # one untimed generation
        reset()
    stream.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"{S}-step graph captured ({R} cache sets in turn); timing it")
    e0.record(stream)
    dec.dec_graph_launch(graph, stream)
    e1.record(stream)
    stream.synchronize()
    total_ms = e0.elapsed_time(e1)
    dec.dec_graph_destroy(graph)
    lens_end = len_d.cpu().numpy()
    steps_end = step_d.cpu().numpy()
    advanced = bool(np.all(lens_end == 1 + S) and np.all(steps_end == S))
    out_ok = bool(torch.isfinite(o_s).all().item() and torch.isfinite(o_c).all().item())
    tok_h = tok.cpu().numpy()
    tok_ok = bool(np.all(((tok_h >= 0) & (tok_h < w.vocab_valid)) | (tok_h == w.fill_token)))
    total_bytes = sum(configs.valid_kv_bytes(w, np.full(B, min(s + 1, w.self_cap), np.int32), c_len)
                      for s in range(S))
    gbs = total_bytes / (total_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": S,
        "warmup": S, "ms_per_step": round(total_ms / S, 6),
        "us_per_step": round(total_ms * 1e3 / S, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "n_layers": w.n_layers, "batch": B, "heads": w.heads,
                   "head_dim": w.head_dim, "self_len": f"s + 1 at step s = 0..{S - 1}",
                   "self_cap": w.self_cap, "cross_len": [int(x) for x in c_len][:4],
                   "cross_cap": w.cross_cap, "top_k": w.top_k, "cache_sets": R,
                   "valid_kv_bytes_total": int(total_bytes),
                   "schedule": (f"decode loop: one graph of {S} steps (dec_kv_append, "
                                f"dec_attn_step, dec_sample_topk_advance: three nodes per "
                                f"step; the steps on {R} cache sets in turn)"
                                if a.separate_append else
                                f"decode loop: one graph of {S} steps (dec_attn_step_append: "
                                f"the current token's rows appended and attended in one "
                                f"launch; dec_sample_topk_advance: sampling and the length "
                                f"and step advance in one launch; the steps on {R} cache "
                                f"sets in turn)"),
                   "uniforms": ("drawn by each sampler launch (Philox4x64-10 in the launch)"
                                if a.draw_in_sampler else
                                f"the generation's {S} x {B} x {w.n_codebooks} Philox4x64-10 "
                                f"uniforms drawn in one dec_philox_uniforms launch at its "
                                f"start (inside the timed graph); step s reads block s")},
        "total_ms": round(total_ms, 3),
        "total_ms_at_70pct_of_peak": round(total_bytes / (0.7 * HBM_PEAK_GBS * 1e9) * 1e3, 3),
        "roofline": {"bound": "hbm", "kernel": "whole step (append + attention, sampler + advance)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "checks": {"outputs_finite": out_ok, "tokens_in_range": tok_ok,
                   "lengths_and_steps_advanced": advanced},
    }
    log(f"{S} steps in {total_ms:.3f} ms ({total_ms * 1e3 / S:.2f} us/step)")
    print(json.dumps(result), flush=True)
    return 0 if (out_ok and tok_ok and advanced) else 1


def calibrate(a):
    """Streaming-read ceilings and the per-node cost of a captured graph."""
    import torch
    import autoregressive_audio_token_amd as dec
    from workloads import configs, gen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)
    w = configs.BY_NAME[a.workload]
    valid = configs.valid_kv_bytes(w, *gen.lengths(w))
    reads = []
    for label, nbytes, pool, n in (("4 MiB, one buffer (cache-resident)", 4 << 20, 0, 2000),
                                   (f"{w.name} valid K/V bytes, rotating buffers", valid,
                                    1 << 30, 200),
                                   ("4 GiB, one buffer", 4 << 30, 0, 10)):
        us, gbs, sets = read_probe(dec, torch, nbytes, dev, stream, n, pool)
        reads.append({"what": label, "bytes": nbytes, "buffers": sets, "avg_launch_us": round(us, 3),
                      "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)})
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nodes = {}
    for n in (1, 49):
        with torch.cuda.stream(stream):
            dec.dec_graph_begin(stream)
            for _ in range(n):
                dec.dec_probe_empty(stream)
            g = dec.dec_graph_end(stream)
            dec.dec_graph_launch(g, stream)
        stream.synchronize()
        reps = 200
        e0.record(stream)
        for _ in range(reps):
            dec.dec_graph_launch(g, stream)
        e1.record(stream)
        stream.synchronize()
        dec.dec_graph_destroy(g)
        nodes[n] = e0.elapsed_time(e1) * 1e3 / reps
    print(json.dumps({"mode": "calibration", "read_kernel": "probe_read_kernel (dec_probe_read)",
                      "reads": reads, "empty_graph_us": {"1 node": round(nodes[1], 3),
                                                         "49 nodes": round(nodes[49], 3)},
                      "us_per_extra_node": round((nodes[49] - nodes[1]) / 48, 3),
                      "timing": "HIP events around replays of captured graphs"}), flush=True)
    return 0


KERNEL_SOURCES = ("attn_decode.hip", "dec_kernels.h", "dec_common.h")


def kernel_sources_sha256():
    """Hash of the attention kernel's sources: counter readings taken on other
    sources no longer describe the kernel."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "autoregressive_audio_token_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary of this
    workload (FETCH_SIZE + WRITE_SIZE, each scaled by the plain-copy calibration),
    or None with the reason when there is none or the kernel changed since."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"attn_decode_{workload}_counters.md")
    if not os.path.exists(path):
        return None, "no counter summary for this workload"
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic-json: "):
                rec = json.loads(line[len("traffic-json: "):])
    if rec is None:
        return None, "counter summary has no traffic-json line"
    if rec.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None, "kernel sources changed since the counters were taken"
    return rec, "counters match the current kernel sources"


def heads_bench(a, w):
    """The merged 9-codebook LM head [B, D] x [9 x 1089, D] on the last position (and the
    merged embedding sum), each timed as a captured graph of back-to-back launches over
    rotating weight sets."""
    import numpy as np
    import torch
    import autoregressive_audio_token_amd as dec
    from workloads import configs, gen, device as wdev

    dev = torch.device("cuda:0")
    if a.batch > 0:
        w = dataclasses.replace(w, batch=a.batch)
    D, B, n_cb = a.d_model or configs.D_MODEL, w.batch, w.n_codebooks
    V, S = w.vocab_valid, w.vocab_stride
    alg = n_cb * V * D * 2 + B * D * 2 + B * n_cb * V * 4       # W valid rows, h, logits
    w_alloc = n_cb * S * D * 2
    R = max(2, math.ceil((1 << 30) / w_alloc))
    h = wdev.to_device(gen.hidden(w, D), dev)
    W0 = wdev.to_device(gen.lm_head_weights(w, D), dev)
    Ws = [W0] + [torch.empty_like(W0).copy_(W0) for _ in range(R - 1)]
    E = wdev.to_device(gen.embedding_table(w, D), dev)
    toks = torch.from_numpy(np.random.default_rng(1).integers(0, V, (B, n_cb)).astype(np.int32)).to(dev)
    logits = torch.empty((B, n_cb, S), dtype=torch.float32, device=dev)
    x = torch.empty((B, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    n_k = max(R, a.kernel_launches)

    def timed(fn):
        with torch.cuda.stream(stream):
            for i in range(R):
                fn(i)
            stream.synchronize()
            dec.dec_graph_begin(stream)
            for i in range(n_k):
                fn(i)
            g = dec.dec_graph_end(stream)
            dec.dec_graph_launch(g, stream)
        stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            dec.dec_graph_launch(g, stream)
        e1.record(stream)
        stream.synchronize()
        dec.dec_graph_destroy(g)
        return e0.elapsed_time(e1) * 1e3 / (3 * n_k)

    head_us = timed(lambda i: dec.dec_lm_head(h, Ws[i % R], logits, B, D, n_cb, V, S, stream))
    kernel_us = {}
    for name, code in (("vector_alu", 1), ("mfma", 2)):   # each kernel alone, for comparison
        dec.dec_tuning_set(head_kernel=code)
        kernel_us[name] = timed(
            lambda i: dec.dec_lm_head(h, Ws[i % R], logits, B, D, n_cb, V, S, stream))
    dec.dec_tuning_set()
    head_us = timed(lambda i: dec.dec_lm_head(h, Ws[i % R], logits, B, D, n_cb, V, S, stream))
    path = "vector_alu" if B <= 2 else "mfma"   # the library's choice at this batch size
    emb_us = timed(lambda i: dec.dec_embed_sum(toks, E, x, B, n_cb, S, D, stream))
    ok = bool(torch.isfinite(logits[:, :, :V]).all().item() and torch.isfinite(x).all().item())
    achieved = alg / (head_us * 1e-6) / 1e9
    # the measured ceiling: a plain streaming read of the same byte count in one launch
    probe_bytes = -(-alg // 16) * 16
    probe_us, probe_gbs, probe_sets = read_probe(dec, torch, probe_bytes, dev, stream, n_k)
    result = {
        "metric": "merged LM head: algorithmic HBM GB/s (weights, hidden state, logits)",
        "value": round(achieved, 1), "unit": "GB/s", "n_gpus": 1, "steps": 3 * n_k,
        "warmup": n_k, "ms_per_step": round(head_us * 1e-3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "d_model": D, "codebooks": n_cb,
                   "vocab": V, "vocab_stride": S, "weight_sets": R,
                   "algorithmic_bytes_per_launch": alg},
        "roofline": {"bound": "hbm",
                     "kernel": ("lm_head_kernel" if path == "vector_alu" else
                                "lm_head_mfma_kernel") + " (dec_lm_head)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "measured_read_gbs": round(probe_gbs, 1),
                     "frac_of_measured": round(achieved / probe_gbs, 4),
                     "measured_read_method": f"dec_probe_read over {probe_bytes} bytes in one "
                                             f"launch, captured graph over {probe_sets} rotating "
                                             f"buffers, {probe_us:.3f} us per launch",
                     "avg_launch_us": round(head_us, 3),
                     "avg_launch_us_method": f"HIP events around a captured graph of {n_k} "
                                             f"launches, 3 replays"},
        "lm_head_path": path,
        "vector_alu_kernel_us": round(kernel_us["vector_alu"], 3),
        "mfma_kernel_us": round(kernel_us["mfma"], 3),
        "embed_sum_us": round(emb_us, 3),
        "checks": {"outputs_finite": ok},
    }
    print(json.dumps(result), flush=True)
    return 0 if ok else 1


def copy_calibration(mib):
    """A plain elementwise copy (bitwise NOT of int32, read n bytes, write n
    bytes) whose FETCH_SIZE / WRITE_SIZE readings scale the attention's."""
    import torch
    dev = torch.device("cuda:0")
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.bitwise_not(a, out=b)
    torch.cuda.synchronize()
    ok = bool((b[:: max(1, n // 4096)] == -2).all().item())
    print(json.dumps({"mode": "copy-calibration", "bytes_read_per_launch": n * 4,
                      "bytes_written_per_launch": n * 4, "launches": 5,
                      "kernel": "torch bitwise_not int32 (elementwise)", "ok": ok}), flush=True)
    return 0 if ok else 1


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, seconds):
    """The oracle, as it stands, on whole decode steps of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attn as oattn, sampling as osamp
    from workloads import configs, gen

    s_len, c_len = gen.lengths(w)
    q = {k: gen.queries(w, k) for k in ("self", "cross")}
    lens = {"self": s_len, "cross": c_len}
    rows = {}
    for kind in ("self", "cross"):
        for layer in range(w.n_layers):
            for b in range(w.batch):
                n = int(lens[kind][b])
                rows[kind, layer, b] = (gen.kv_rows(w, kind, "k", layer, b, n),
                                        gen.kv_rows(w, kind, "v", layer, b, n))
    lg, u, T = gen.logits(w), gen.uniforms(w), gen.temperatures(w)
    dec16 = oattn.bf16_bits_to_f64 if w.dtype == "bf16" else (lambda x: x.astype(np.float64))

    tasks = [(kind, layer, b) for kind in ("self", "cross") for layer in range(w.n_layers)
             for b in range(w.batch)]

    def attend(task):  # every head of one (segment, layer, sequence)
        kind, layer, b = task
        K, V = rows[task]
        n = int(lens[kind][b])
        for h in range(w.heads):
            oattn.attend_one(dec16(q[kind][layer, b, h]), dec16(K[h]), dec16(V[h]), n, w.scale)

    def one_step():
        for t in tasks:
            attend(t)
        osamp.sample(lg, w.vocab_valid, T, w.top_k, u, None, w.fill_token)

    times, t0 = [], time.perf_counter()
    with threadpool_limits(1):  # one thread, BLAS included
        while len(times) < 10 or time.perf_counter() - t0 < seconds:
            s = time.perf_counter()
            one_step()
            times.append(time.perf_counter() - s)
    valid = configs.valid_kv_bytes(w, s_len, c_len)
    med = statistics.median(times)
    return {"value": round(valid / med / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{len(times)} whole decode steps of {w.name} (all layers, self+cross "
                      f"attention over the valid prefixes, then the sampler), float64 NumPy, "
                      f"one thread; value from the median step time",
            "us_per_step": round(med * 1e6, 1),
            "us_per_step_mean": round(sum(times) / len(times) * 1e6, 1),
            "host_cpu": _cpu_model(),
            "host_cores_visible": len(os.sched_getaffinity(0)),
            "host_cpu_count": os.cpu_count()}


def cpu_baseline_all_cores(w, seconds):
    """The oracle, as it stands, on every host core: worker processes, forked before this
    process makes any GPU call, each own a share of a step's (segment, layer, sequence)
    attention tasks (the last also runs the sampler) and build their own inputs.  A step
    starts every worker at a barrier and ends when the last one is done; BLAS runs one
    thread per worker.  Returns None if a worker fails."""
    import multiprocessing as mp
    import threading
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attn as oattn, sampling as osamp
    from workloads import configs, gen

    s_len, c_len = gen.lengths(w)
    lens = {"self": s_len, "cross": c_len}
    tasks = [(kind, layer, b) for kind in ("self", "cross") for layer in range(w.n_layers)
             for b in range(w.batch)]
    n_workers = max(1, min(len(os.sched_getaffinity(0)), len(tasks)))
    ctx = mp.get_context("fork")
    ready, start, done = (ctx.Barrier(n_workers + 1) for _ in range(3))
    stop = ctx.Value("i", 0)
    limit = 300.0  # seconds any barrier may wait: a dead worker breaks the barriers

    def work(i):
        try:
            share = tasks[i::n_workers]
            q = {k: gen.queries(w, k) for k in ("self", "cross")}
            rows = {t: (gen.kv_rows(w, t[0], "k", t[1], t[2], int(lens[t[0]][t[2]])),
                        gen.kv_rows(w, t[0], "v", t[1], t[2], int(lens[t[0]][t[2]])))
                    for t in share}
            sampler = i == n_workers - 1
            if sampler:
                lg, u, T = gen.logits(w), gen.uniforms(w), gen.temperatures(w)
            dec16 = (oattn.bf16_bits_to_f64 if w.dtype == "bf16"
                     else (lambda x: x.astype(np.float64)))
            with threadpool_limits(1):
                ready.wait(limit)
                while True:
                    start.wait(limit)
                    if stop.value:
                        break
                    for kind, layer, b in share:
                        K, V = rows[kind, layer, b]
                        for h in range(w.heads):
                            oattn.attend_one(dec16(q[kind][layer, b, h]), dec16(K[h]),
                                             dec16(V[h]), int(lens[kind][b]), w.scale)
                    if sampler:
                        osamp.sample(lg, w.vocab_valid, T, w.top_k, u, None, w.fill_token)
                    done.wait(limit)
        except Exception:
            for bar in (ready, start, done):
                bar.abort()
        os._exit(0)  # no interpreter teardown in a forked child

    procs = [ctx.Process(target=work, args=(i,), daemon=True) for i in range(n_workers)]
    for p in procs:
        p.start()
    times = []
    try:
        ready.wait(limit)
        t0 = time.perf_counter()
        while len(times) < 10 or time.perf_counter() - t0 < seconds:
            s = time.perf_counter()
            start.wait(limit)
            done.wait(limit)
            times.append(time.perf_counter() - s)
        stop.value = 1
        start.wait(limit)
    except threading.BrokenBarrierError:
        times = []
    for p in procs:
        p.join(30)
        if p.is_alive():
            p.kill()
    if not times:
        return None
    valid = configs.valid_kv_bytes(w, s_len, c_len)
    med = statistics.median(times)
    return {"value": round(valid / med / 1e9, 4), "unit": "GB/s", "cores": n_workers,
            "kind": "oracle",
            "sample": f"{len(times)} whole decode steps of {w.name}, float64 NumPy, the step's "
                      f"{len(tasks)} (segment, layer, sequence) tasks shared by {n_workers} "
                      f"worker processes (one thread each; the last also samples); value from "
                      f"the median step time",
            "us_per_step": round(med * 1e6, 1),
            "us_per_step_mean": round(sum(times) / len(times) * 1e6, 1)}


def main(argv=None):
    a = parse(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}): the library has "
              "no multi-GPU path; the work is sized for a single MI355X.", file=sys.stderr)
        return 2
    if a.copy_mib > 0:
        return copy_calibration(a.copy_mib)
    if a.calibrate:
        return calibrate(a)
    if a.decode_loop:
        return decode_loop(a)

    import numpy as np
    import torch
    import autoregressive_audio_token_amd as dec
    from workloads import configs, gen, device as wdev

    w = configs.BY_NAME[a.workload]
    if a.heads:
        return heads_bench(a, w)
    if a.head_dim != w.head_dim:     # the same model width in heads of a.head_dim
        w = dataclasses.replace(w, heads=w.heads * w.head_dim // a.head_dim, head_dim=a.head_dim,
                                scale=a.head_dim ** -0.5, qkv_std=a.head_dim ** -0.5)
    top_k = a.top_k if a.top_k > 0 else w.top_k
    ex_attn = a.cross_mask > 0 or a.out_bf16
    ex_samp = top_k > 64 or a.logits_bf16
    model = a.schedule == "model"
    if model and (ex_attn or a.paged):
        print("--schedule model goes with the static caches and fp32 outputs", file=sys.stderr)
        return 2
    plain = not (ex_attn or ex_samp or a.paged or a.head_dim != 64 or a.top_k or model or
                 a.attn_chunk)
    if a.attn_chunk:
        dec.dec_tuning_set(attn_chunk_keys=a.attn_chunk)
    all_cores = None
    if not a.no_cpu_baseline:  # its worker processes are forked before any GPU call
        print("[bench] timing the oracle on all host cores", file=sys.stderr, flush=True)
        all_cores = cpu_baseline_all_cores(w, a.cpu_seconds)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s_len, c_len = gen.lengths(w)
    valid = configs.valid_kv_bytes(w, s_len, c_len)
    mask_d, mask_words, mask_note = None, 0, None
    if a.cross_mask > 0:
        # seeded boolean description mask; algorithmic bytes count attended keys only
        rng = np.random.default_rng(777)
        if a.mask_runs > 0:
            runs = rng.random((w.batch, -(-w.cross_cap // a.mask_runs))) < a.cross_mask
            mask = np.repeat(runs, a.mask_runs, axis=1)[:, :w.cross_cap]
        else:
            mask = rng.random((w.batch, w.cross_cap)) < a.cross_mask
        mask_words = 2 * ((w.cross_cap + 63) // 64)
        padded = np.zeros((w.batch, mask_words * 32), bool)
        padded[:, :w.cross_cap] = mask
        packed = np.ascontiguousarray(np.packbits(padded, axis=1, bitorder="little")).view(np.uint32)
        mask_d = torch.from_numpy(packed.copy()).to(dev)
        attended = sum(int(mask[b, :int(c_len[b])].sum()) for b in range(w.batch))
        row = w.head_dim * (2 if w.dtype == "bf16" else 4)
        cross_all = sum(int(n) for n in c_len) * w.n_layers * w.heads * row * 2
        valid = valid - cross_all + attended * w.n_layers * w.heads * row * 2
        mask_note = (f"keep probability {a.cross_mask}, runs of {a.mask_runs or 1} keys: "
                     f"{attended} of {int(sum(c_len))} description keys attended")
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)
    log(f"workload {w.name}: staging inputs")
    d = wdev.step_inputs(w, dev)
    R = a.sets if a.sets > 0 else max(2, math.ceil((1 << 30) / valid))
    big = ("k_self", "v_self", "k_cross", "v_cross")
    sets = [{k: d[k] for k in big}]
    for _ in range(R - 1):
        sets.append({k: torch.empty_like(d[k]).copy_(d[k]) for k in big})
    static_bytes = sum(d[k].numel() * d[k].element_size() for k in big)
    code = dec.DEC_BF16 if w.dtype == "bf16" else dec.DEC_F32
    nb = dec.dec_attn_workspace_bytes(w.n_layers, w.batch, w.heads, w.head_dim, w.self_cap,
                                      w.cross_cap)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    o_s = torch.empty((w.n_layers, w.batch, w.heads, w.head_dim),
                      dtype=torch.bfloat16 if a.out_bf16 else torch.float32, device=dev)
    o_c = torch.empty_like(o_s)
    logits = d["logits"].to(torch.bfloat16) if a.logits_bf16 else d["logits"]
    tok = torch.empty((w.batch, w.n_codebooks), dtype=torch.int32, device=dev)
    step_t = d["step"] if w.delay else None
    stream = torch.cuda.Stream(device=dev)

    if a.paged:
        # every cache set's self cache scattered over a pool: logical block i of sequence b
        # lives in physical block table[b, i]; the pool holds one spare block per sequence
        bs = a.paged
        mb = w.self_cap // bs
        pool_blocks = w.batch * (mb + 1)
        perm = np.random.default_rng(12345).permutation(pool_blocks)[:w.batch * mb]
        table_h = perm.reshape(w.batch, mb).astype(np.int32)
        table = torch.from_numpy(table_h).to(dev)
        idx = torch.from_numpy(table_h.reshape(-1)).to(dev).long()
        for st in sets:
            for which in ("k_self", "v_self"):
                src = st[which]                       # [NL, B, H, L_cap, hd]
                pool = torch.full((w.n_layers, pool_blocks, w.heads, bs, w.head_dim), float("nan"),
                                  dtype=src.dtype, device=dev)
                blocks = src.view(w.n_layers, w.batch, w.heads, mb, bs, w.head_dim)
                blocks = blocks.permute(0, 1, 3, 2, 4, 5).reshape(
                    w.n_layers, w.batch * mb, w.heads, bs, w.head_dim)
                pool[:, idx] = blocks
                st[which] = pool
        torch.cuda.synchronize()

    def attn(st, s):
        if ex_attn and a.paged:          # a paged self cache with the widenings
            dec.dec_attn_step_paged_ex(d["q_self"], st["k_self"], st["v_self"], table, d["len"],
                                       a.paged, pool_blocks, w.self_cap // a.paged, o_s,
                                       d["q_cross"], st["k_cross"], st["v_cross"], d["enc_len"],
                                       mask_d, mask_words, w.cross_cap, o_c, w.n_layers, w.batch,
                                       w.heads, w.head_dim, code,
                                       dec.DEC_BF16 if a.out_bf16 else dec.DEC_F32, w.scale, ws,
                                       nb, s)
            return
        if model:                        # one self and one cross launch per layer
            for l in range(w.n_layers):
                dec.dec_attn_self(d["q_self"][l], st["k_self"][l], st["v_self"][l], d["len"],
                                  o_s[l], 1, w.batch, w.heads, w.self_cap, w.head_dim, code,
                                  w.scale, ws, nb, s)
                dec.dec_attn_cross(d["q_cross"][l], st["k_cross"][l], st["v_cross"][l],
                                   d["enc_len"], o_c[l], 1, w.batch, w.heads, w.cross_cap,
                                   w.head_dim, code, w.scale, ws, nb, s)
            return
        if ex_attn:
            dec.dec_attn_step_ex(d["q_self"], st["k_self"], st["v_self"], d["len"], w.self_cap,
                                 o_s, d["q_cross"], st["k_cross"], st["v_cross"], d["enc_len"],
                                 mask_d, mask_words, w.cross_cap, o_c, w.n_layers, w.batch,
                                 w.heads, w.head_dim, code,
                                 dec.DEC_BF16 if a.out_bf16 else dec.DEC_F32, w.scale, ws, nb, s)
            return
        if a.paged:
            dec.dec_attn_step_paged(d["q_self"], st["k_self"], st["v_self"], table, d["len"],
                                    a.paged, pool_blocks, w.self_cap // a.paged, o_s, d["q_cross"],
                                    st["k_cross"], st["v_cross"], d["enc_len"], w.cross_cap, o_c,
                                    w.n_layers, w.batch, w.heads, w.head_dim, code, w.scale, ws,
                                    nb, s)
            return
        dec.dec_attn_step(d["q_self"], st["k_self"], st["v_self"], d["len"], w.self_cap, o_s,
                          d["q_cross"], st["k_cross"], st["v_cross"], d["enc_len"], w.cross_cap,
                          o_c, w.n_layers, w.batch, w.heads, w.head_dim, code, w.scale, ws, nb,
                          s)

    def sample(s):
        if ex_samp:
            dec.dec_sample_topk_ex(logits, dec.DEC_BF16 if a.logits_bf16 else dec.DEC_F32,
                                   w.batch, w.n_codebooks, w.vocab_valid, w.vocab_stride,
                                   d["temperature"], top_k, d["uniforms"], 0, step_t,
                                   w.fill_token, tok, None, None, s)
            return
        dec.dec_sample_topk(logits, w.batch, w.n_codebooks, w.vocab_valid, w.vocab_stride,
                            d["temperature"], top_k, d["uniforms"], step_t, w.fill_token, tok,
                            None, None, s)

    torch.cuda.synchronize()
    if a.eager:
        with torch.cuda.stream(stream):
            dec.dec_attn_workspace_init(ws, nb, stream)
            for i in range(a.warmup + a.steps):
                attn(sets[i % R], stream)
                sample(stream)
        stream.synchronize()
        print(json.dumps({"mode": "eager", "workload": w.name, "steps": a.warmup + a.steps,
                          "cache_sets": R, "valid_kv_bytes_per_step": valid,
                          "outputs_finite": bool(torch.isfinite(o_s).all().item())}),
              flush=True)
        return 0
    # Exactly `warmup` untimed steps, then exactly `steps` timed ones, each step on the next
    # cache set in rotation (no set is read twice within R steps, so a step finds its K/V
    # bytes in HBM, not in a cache).  Each runs as one captured graph.  `value` comes from
    # HIP events around the timed graph's launch.  A second run of as many steps, after the
    # timed one, has dec_probe_clock nodes at the edges of min(10, steps) blocks of
    # near-equal size (one node each); the per-block step times come from one XCD's clock.
    def split(total, parts):
        q, r = divmod(total, parts)
        return [q + 1] * r + [q] * (parts - r)

    def capture(first, sizes, clocks=None):
        with torch.cuda.stream(stream):
            dec.dec_graph_begin(stream)
            pos = first
            if clocks is not None:
                dec.dec_probe_clock(clocks[0], stream)
            for i, n in enumerate(sizes):
                for _ in range(n):
                    attn(sets[pos % R], stream)
                    sample(stream)
                    pos += 1
                if clocks is not None:
                    dec.dec_probe_clock(clocks[i + 1], stream)
            return dec.dec_graph_end(stream)

    steps = a.steps
    n_blocks = min(10, steps)
    timed = split(steps, n_blocks)
    clocks = torch.zeros((n_blocks + 1, 16), dtype=torch.int64, device=dev)
    warm_graph = capture(0, [a.warmup]) if a.warmup > 0 else None
    timed_graph = capture(a.warmup, [steps])
    # the same number of steps again, after the timed run and outside it, with clock nodes at
    # the block edges (each node costs about an empty graph node, so they stay out of `value`)
    block_graph = capture(a.warmup + steps, timed, clocks)
    with torch.cuda.stream(stream):
        dec.dec_attn_workspace_init(ws, nb, stream)
    log(f"{R} cache sets; {a.warmup} warm-up and {steps} timed steps captured ({n_blocks} "
        f"clocked blocks in a separate run)")
    if warm_graph is not None:
        dec.dec_graph_launch(warm_graph, stream)
    stream.synchronize()
    torch.cuda.synchronize()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e_start.record(stream)
    dec.dec_graph_launch(timed_graph, stream)
    e_end.record(stream)
    stream.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e_start.elapsed_time(e_end) / steps
    dec.dec_graph_launch(block_graph, stream)
    stream.synchronize()
    ck = clocks.cpu().numpy()
    xcd = next(x for x in range(ck.shape[1]) if np.all(ck[:, x] > 0))  # one XCD's clock
    blk_us = sorted(float(ck[i + 1, xcd] - ck[i, xcd]) * 0.01 / timed[i] for i in range(n_blocks))
    for g in (warm_graph, timed_graph, block_graph):
        if g is not None:
            dec.dec_graph_destroy(g)
    out_ok = bool(torch.isfinite(o_s).all().item() and torch.isfinite(o_c).all().item())
    tok_h = tok.cpu().numpy()
    tok_ok = bool(np.all((tok_h >= 0) & (tok_h < w.vocab_valid) | (tok_h == w.fill_token)))

    # roofline leg: the attention kernel alone.  A captured graph of n_k
    # back-to-back launches (rotating cache sets) is timed with one event pair,
    # so the average carries only the graph's inter-node gap; per-launch event
    # pairs are reported beside it.
    n_k = max(R, a.kernel_launches)
    with torch.cuda.stream(stream):
        dec.dec_graph_begin(stream)
        for i in range(n_k):
            attn(sets[i % R], stream)
        kgraph = dec.dec_graph_end(stream)
        dec.dec_graph_launch(kgraph, stream)        # warm
    stream.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k_reps = 3
    k0.record(stream)
    for _ in range(k_reps):
        dec.dec_graph_launch(kgraph, stream)
    k1.record(stream)
    stream.synchronize()
    k_us = k0.elapsed_time(k1) * 1e3 / (k_reps * n_k)
    dec.dec_graph_destroy(kgraph)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_k)]
    with torch.cuda.stream(stream):
        for i in range(n_k):
            evs[i][0].record(stream)
            attn(sets[i % R], stream)
            evs[i][1].record(stream)
    stream.synchronize()
    per = sorted(s0.elapsed_time(s1) * 1e3 for s0, s1 in evs)        # microseconds
    pair_us = sum(per) / len(per)
    achieved = valid / (k_us * 1e-6) / 1e9
    # the measured ceiling: a plain streaming read of the same byte count in one launch
    probe_us, probe_gbs, probe_sets = read_probe(dec, torch, valid, dev, stream, n_k)
    # the sampler alone: a captured graph of n_k launches
    with torch.cuda.stream(stream):
        dec.dec_graph_begin(stream)
        for _ in range(n_k):
            sample(stream)
        sgraph = dec.dec_graph_end(stream)
        dec.dec_graph_launch(sgraph, stream)        # warm
    stream.synchronize()
    k0.record(stream)
    for _ in range(k_reps):
        dec.dec_graph_launch(sgraph, stream)
    k1.record(stream)
    stream.synchronize()
    samp_us = k0.elapsed_time(k1) * 1e3 / (k_reps * n_k)
    dec.dec_graph_destroy(sgraph)
    traffic_rec, traffic_why = counter_traffic(w.name)
    if not plain:
        traffic_rec, traffic_why = None, "counters describe the default configuration only"
    if model:
        traffic_rec, traffic_why = None, "counters describe the stacked launch only"
    attn_entry = ("dec_attn_self + dec_attn_cross per layer" if model else
                  "dec_attn_step_paged_ex" if ex_attn and a.paged else
                  "dec_attn_step_ex" if ex_attn else
                  "dec_attn_step_paged" if a.paged else "dec_attn_step")
    attn_launches = 2 * w.n_layers if model else 1
    samp_entry = "dec_sample_topk_ex" if ex_samp else "dec_sample_topk"

    result = {
        "metric": METRIC,
        "value": round(valid / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "us_per_step_blocks": {"blocks": n_blocks, "steps_per_block": [min(timed), max(timed)],
                               "median": round(blk_us[len(blk_us) // 2], 3),
                               "min": round(blk_us[0], 3), "max": round(blk_us[-1], 3),
                               "clock": f"XCD {xcd}'s 100 MHz clock, read by dec_probe_clock "
                                        f"nodes at the block edges of a second run of the same "
                                        f"number of steps, after the timed one"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "n_layers": w.n_layers, "batch": w.batch, "heads": w.heads,
            "head_dim": w.head_dim, "self_len": [int(x) for x in s_len][:4],
            "self_cap": w.self_cap, "cross_len": [int(x) for x in c_len][:4],
            "cross_cap": w.cross_cap, "codebooks": w.n_codebooks, "vocab": w.vocab_valid,
            "vocab_stride": w.vocab_stride, "top_k": top_k, "accumulate": "f32",
            "valid_kv_bytes_per_step": valid, "cache_sets": R,
            "static_cache_bytes_per_set": static_bytes,
            "kv_layout": (f"self cache paged, {a.paged} keys per block" if a.paged
                          else "static caches"),
            "schedule": (f"model-shaped: the timed steps as one hipGraph; step = {attn_entry} "
                         f"({attn_launches} launches) + {samp_entry}" if model else
                         f"the timed steps as one hipGraph; step = {attn_entry} (self+cross, "
                         f"all layers, one launch) + {samp_entry}"),
            "variant": {"head_dim": w.head_dim, "cross_mask": mask_note,
                        "attention_outputs": "bf16" if a.out_bf16 else "f32",
                        "logits": "bf16" if a.logits_bf16 else "f32", "top_k": top_k,
                        "attn_chunk_keys": a.attn_chunk or "chosen per launch"},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": f"attn_decode_kernel ({attn_entry})",
            "launches_per_step": attn_launches,
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_rec["hbm_bytes_per_launch"] if traffic_rec else None,
            "traffic_detail": {"status": traffic_why, **({k: traffic_rec[k] for k in (
                "hbm_read_bytes_per_launch", "hbm_write_bytes_per_launch", "fetch_scale",
                "write_scale", "ratio_to_algorithmic")} if traffic_rec else {})},
            "avg_launch_us": round(k_us, 3),
            "avg_launch_us_method": (f"HIP events around a captured graph of {n_k} attention "
                                     f"steps ({attn_launches} launches each), {k_reps} replays"
                                     if model else
                                     f"HIP events around a captured graph of {n_k} launches, "
                                     f"{k_reps} replays"),
            "event_pair_avg_us": round(pair_us, 3),
            "event_pair_median_us": round(per[len(per) // 2], 3), "launches": n_k,
            "algorithmic_bytes_per_launch": valid,
            "measured_read_gbs": round(probe_gbs, 1),
            "frac_of_measured": round(achieved / probe_gbs, 4),
            "measured_read_method": f"dec_probe_read (a plain streaming read) over the same "
                                    f"{valid} bytes in one launch: a captured graph of "
                                    f"{max(n_k, probe_sets)} launches over {probe_sets} rotating "
                                    f"buffers, {probe_us:.3f} us per launch",
        },
        "sampler": {"kernel": f"sample_topk_kernel ({samp_entry})", "top_k": top_k,
                    "avg_launch_us": round(samp_us, 3),
                    "avg_launch_us_method": f"HIP events around a captured graph of {n_k} "
                                            f"launches, {k_reps} replays"},
        "checks": {"outputs_finite": out_ok, "tokens_in_range": tok_ok},
        "host_wall_s": round(wall, 4),
    }
    log(f"{ms_per_step * 1e3:.2f} us/step; attention launch {k_us:.2f} us (pairs {pair_us:.2f})")
    if not a.no_cpu_baseline:
        log("timing the oracle on the host")
        result["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
        result["cpu_baseline"]["all_cores"] = all_cores
    print(json.dumps(result), flush=True)
    return 0 if (out_ok and tok_ok) else 1


if __name__ == "__main__":
    sys.exit(main())
