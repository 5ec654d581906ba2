"""bench.py's output line on the GPU: one JSON object with the contract's fields, on a short run
of the smallest batch-1 workload (the timings themselves are not checked)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def test_bench_prints_one_contract_line():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "llama-16k",
                        "--steps", "20", "--warmup", "4", "--no-dense", "--no-builder", "--quiet"],
                       capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline", "step_spread", "kernels", "keys_scored_per_s",
              "hamming_scored_per_s"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 4
    assert d["higher_is_better"] is False and d["unit"] == "us/step/layer"
    assert abs(d["ms_per_step"] * 1e3 - d["value"]) < 1e-6 * max(1.0, d["value"]) + 1e-3
    assert d["config"]["workload"] and d["config"]["seq_len"] == 16384
    # 32 query heads x 128 kept pages (keep 1/8 of 1024) x 16 tokens per step
    assert abs(d["hamming_scored_per_s"] * d["ms_per_step"] * 1e-3 / (32 * 128 * 16) - 1) < 1e-3
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["kernel"] in d["kernels"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == len(os.sched_getaffinity(0))
    assert cb["value"] > 0 and cb["single_thread_value"] > 0 and cb["sample"]
    assert cb["builder_value"] > 0 and cb["builder_single_thread_value"] > 0
    sp = d["step_spread"]
    assert sp["p10_us"] <= sp["p50_us"] <= sp["p90_us"]
    # the kernels a batch-1 step launches, each timed
    assert set(d["kernels"]) == {"prep", "page_bound", "select", "sparse_attn", "combine"}
    assert all(v["avg_us"] > 0 for v in d["kernels"].values())
