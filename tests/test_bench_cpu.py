"""Host-side pieces of bench.py: the one-GPU guard and the counter-traffic record."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counter_record_parses_and_is_consistent():
    rec, why = bench.counter_traffic("long_description")
    if rec is None:
        # the summary exists; only a kernel change may disable it
        assert why == "kernel sources changed since the counters were taken"
        path = os.path.join(ROOT, "profiles", "attn_decode_long_description_counters.md")
        line = [ln for ln in open(path) if ln.startswith("traffic-json: ")][-1]
        rec = json.loads(line[len("traffic-json: "):])
    # scaled counters add up, and each scale is what the copy calibration gives
    kib = 1024
    assert abs(rec["fetch_scale"] - rec["copy_calibration_bytes"]
               / (rec["copy_fetch_size_kib"] * kib)) < 1e-4
    assert abs(rec["write_scale"] - rec["copy_calibration_bytes"]
               / (rec["copy_write_size_kib"] * kib)) < 1e-4
    rd = rec["fetch_size_kib_per_dispatch"] * kib * rec["fetch_scale"]
    wr = rec["write_size_kib_per_dispatch"] * kib * rec["write_scale"]
    assert abs(rec["hbm_read_bytes_per_launch"] - rd) / rd < 1e-4
    assert abs(rec["hbm_write_bytes_per_launch"] - wr) < 1
    assert rec["hbm_bytes_per_launch"] == (rec["hbm_read_bytes_per_launch"]
                                           + rec["hbm_write_bytes_per_launch"])


def test_unknown_workload_has_no_traffic():
    rec, why = bench.counter_traffic("no_such_workload")
    assert rec is None and "no counter summary" in why


def test_paged_and_widened_options_combine():
    # a paged self cache with a description mask and bf16 outputs: dec_attn_step_paged_ex
    a = bench.parse(["--paged", "64", "--cross-mask", "0.5", "--out-bf16"])
    assert (a.paged, a.cross_mask, a.out_bf16) == (64, 0.5, True)


def test_variant_options_parse():
    a = bench.parse(["--head-dim", "128", "--cross-mask", "0.3", "--mask-runs", "64",
                     "--out-bf16", "--top-k", "250", "--logits-bf16"])
    assert (a.head_dim, a.cross_mask, a.mask_runs, a.out_bf16, a.top_k, a.logits_bf16) == \
        (128, 0.3, 64, True, 250, True)


def test_model_schedule_with_widened_or_paged_attention_is_refused():
    assert bench.main(["--schedule", "model", "--paged", "64"]) == 2
    assert bench.main(["--schedule", "model", "--out-bf16"]) == 2


def test_decode_loop_needs_a_workload_with_steps():
    assert bench.main(["--decode-loop", "--workload", "long_description"]) == 2


def test_measurement_options_parse():
    a = bench.parse(["--schedule", "model", "--decode-loop", "--calibrate"])
    assert (a.schedule, a.decode_loop, a.calibrate) == ("model", True, True)
    assert bench.parse([]).schedule == "stacked"


def test_oracle_baseline_reports_the_median_of_at_least_ten_steps():
    from workloads import configs, gen
    r = bench.cpu_baseline(configs.TINY, 0.0)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["unit"] == "GB/s"
    steps = int(r["sample"].split()[0])
    assert steps >= 10
    # value: the valid K/V bytes of one step over the median step time
    s_len, c_len = gen.lengths(configs.TINY)
    valid = configs.valid_kv_bytes(configs.TINY, s_len, c_len)
    assert abs(r["value"] - valid / (r["us_per_step"] * 1e-6) / 1e9) <= 1e-3 * r["value"] + 1e-4
    assert r["host_cores_visible"] >= 1 and r["host_cpu_count"] >= r["host_cores_visible"]
    assert isinstance(r["host_cpu"], str) and r["host_cpu"]


def test_steps_and_warmup_are_validated():
    for argv in (["--steps", "0"], ["--warmup", "-1"]):
        with pytest.raises(SystemExit):
            bench.parse(argv)
    a = bench.parse(["--steps", "20", "--warmup", "5"])
    assert (a.steps, a.warmup) == (20, 5)


def test_oracle_baseline_on_all_cores_runs_whole_steps_in_worker_processes():
    from workloads import configs, gen
    r = bench.cpu_baseline_all_cores(configs.TINY, 0.0)
    assert r is not None, "a worker failed"
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert 1 <= r["cores"] <= len(os.sched_getaffinity(0))
    steps = int(r["sample"].split()[0])
    assert steps >= 10
    s_len, c_len = gen.lengths(configs.TINY)
    valid = configs.valid_kv_bytes(configs.TINY, s_len, c_len)
    assert abs(r["value"] - valid / (r["us_per_step"] * 1e-6) / 1e9) <= 1e-3 * r["value"] + 1e-4


def test_the_default_path_reaches_the_gpu_step_on_a_host_without_one(monkeypatch):
    # everything main() does before its first GPU call (argument checks, the all-cores
    # oracle baseline) runs on the CPU; the GPU step is stubbed to stop there
    import torch
    from workloads import configs
    calls = []
    monkeypatch.setattr(bench, "cpu_baseline_all_cores",
                        lambda w, s: calls.append(w.name) or {"value": 1.0})

    def stop(dev):
        raise RuntimeError("reached the GPU step")
    monkeypatch.setattr(torch.cuda, "set_device", stop)
    with pytest.raises(RuntimeError, match="reached the GPU step"):
        bench.main(["--workload", "tiny", "--cpu-seconds", "0"])
    assert calls == [configs.TINY.name]


def test_attention_chunk_option_parses():
    assert bench.parse(["--attn-chunk", "256"]).attn_chunk == 256
    for bad in ("100", "2048", "96"):
        with pytest.raises(SystemExit):
            bench.parse(["--attn-chunk", bad])
