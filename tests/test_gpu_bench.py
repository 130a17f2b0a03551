"""bench.py end to end on the GPU, in each of its modes with few steps: one JSON line with the metric,
the value, the roofline of the dominant kernel (HIP-event launch times) and, for the default run, the
oracle's CPU baseline on a bounded sample."""
import json
import os
import subprocess
import sys

import pytest

from gpu_helpers import announce, device

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config")


def _bench(*args):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1", *args]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    print(res.stderr[-2000:], flush=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return json.loads(res.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("args", [("--cpu-rows", "256"), ("--no-cpu-baseline", "--sequences", "8"),
                                  ("--no-cpu-baseline", "--mode", "forward"),
                                  ("--no-cpu-baseline", "--mode", "recompute")],
                         ids=["default", "sequences", "forward", "recompute"])
def test_bench_modes_print_the_contract_line(args):
    device()
    announce("bench.py", *args)
    d = _bench(*args)
    for k in KEYS:
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["value"] > 0
    assert d["unit"] == "tokens/s" and d["config"]["workload"] == "llama3_8b_head"
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert 0.0 < r["frac"] < 1.0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert d["peak_bytes"]["workspace"] < d["peak_bytes"]["full_bf16_logits_not_allocated"]
    mp = d["measured_peaks"]
    assert 1000.0 < mp["mfma_bf16_tflops"] <= 2525.0 and 1000.0 < mp["copy_gbs"] <= 8080.0
    assert abs(r["frac_of_measured_peak"] - r["achieved"] / mp["mfma_bf16_tflops"]) < 1e-3
    assert 0.0 < d["mfma_frac_step_of_measured"] < 1.0
    if "--no-cpu-baseline" not in args:
        c = d["cpu_baseline"]
        assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and "256" in c["sample"]
