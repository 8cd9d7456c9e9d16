"""bench.py's optional paths, each run once at small sizes (GPU).

Each case starts bench.py in a child process with a few steps over two cache sets and checks
that it exits cleanly and ends with one JSON record.  The figures are not checked here (the
bench measures them); the point is that every path the bench offers still runs against the
library's entry points and the binding's argument checks.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CASES = {
    "paged": ["--paged", "64"],
    "paged_masked_bf16": ["--paged", "64", "--cross-mask", "0.5", "--out-bf16"],
    "head_dim_128": ["--head-dim", "128"],
    "wide_top_k": ["--top-k", "250"],
    "mask_runs_bf16_out": ["--cross-mask", "0.5", "--mask-runs", "64", "--out-bf16"],
    "bf16_logits": ["--logits-bf16"],
    "model_schedule": ["--schedule", "model"],
    "fixed_chunk": ["--attn-chunk", "256"],
    "eager": ["--eager"],
    "heads": ["--heads"],
    "decode_loop": ["--workload", "long_output", "--decode-loop"],
    "decode_loop_draw_in_sampler": ["--workload", "long_output", "--decode-loop",
                                    "--draw-in-sampler"],
    "calibrate": ["--calibrate"],
}
SMALL = ["--steps", "4", "--warmup", "1", "--sets", "2", "--kernel-launches", "10",
         "--no-cpu-baseline"]


@pytest.mark.gpu
@pytest.mark.parametrize("name", sorted(CASES))
def test_bench_path_runs(name):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), *CASES[name], *SMALL]
    print(f"[bench path] {name}: {' '.join(cmd[2:])}", flush=True)
    res = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert res.returncode == 0, res.stderr[-3000:]
    rec = json.loads(res.stdout.strip().splitlines()[-1])
    assert isinstance(rec, dict) and rec, res.stdout[-2000:]
    if "value" in rec:
        assert rec["value"] > 0, rec
