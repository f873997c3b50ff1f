"""bench.py's output line: one JSON object with the keys, types and internal consistency its readers
rely on (value against ms_per_step, the roofline fraction, the cache mode, the CPU-oracle baseline).
Runs the bench in a child process on the tiny witness workload and on two steps of the headline step.
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric": str, "value": float, "unit": str, "n_gpus": int, "steps": int, "warmup": int,
        "ms_per_step": float, "higher_is_better": bool, "scaling": str, "dtype": str, "data": str,
        "config": dict, "roofline": dict}
ROOFLINE = {"bound": str, "achieved": float, "peak": float, "unit": str, "frac": float}


def run_bench(*args):
    print(f"bench.py {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def check_common(rec, steps, warmup):
    for k, t in KEYS.items():
        assert k in rec and isinstance(rec[k], t), (k, rec.get(k))
    assert rec["n_gpus"] == 1 and rec["steps"] == steps and rec["warmup"] == warmup
    assert rec["higher_is_better"] is True and rec["scaling"] == "weak" and rec["dtype"] == "bf16"
    assert rec["unit"] == "TFLOP/s" and rec["vs_baseline"] is None
    assert "workload" in rec["config"] and "caches" in rec["config"]
    rf = rec["roofline"]
    for k, t in ROOFLINE.items():
        assert k in rf and isinstance(rf[k], t), (k, rf.get(k))
    assert rf["bound"] in ("mfma", "hbm")
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "traffic" in rf
    assert rec["value"] > 0 and rec["ms_per_step"] > 0
    assert rec["per_workload"] and all(w["kernel_ms"] > 0 and w["useful_tflops"] > 0 for w in rec["per_workload"])


def test_witness_workload_with_cpu_baseline():
    rec = run_bench("--workload", "causal_witness_33x47", "--steps", "3", "--warmup", "1", "--cpu-budget", "5")
    check_common(rec, 3, 1)
    # below the ridge: HBM roofline on algorithmic bytes, cold caches by default
    assert rec["roofline"]["bound"] == "hbm" and rec["roofline"]["unit"] == "GB/s"
    assert rec["roofline"]["peak"] == 8000.0
    assert rec["config"]["caches"].startswith("cold")
    cb = rec["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0 and cb["cores"] >= 1
    assert "causal_witness_33x47" in cb["sample"]


def test_headline_step_two_steps():
    rec = run_bench("--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    check_common(rec, 2, 1)
    assert rec["config"]["workload"] == "causal_8k_32k"
    assert [w["name"] for w in rec["per_workload"]] == ["mid_ctx_8k", "long_ctx_32k"]
    rf = rec["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and abs(rf["peak"] - 2516.6) < 1e-6
    assert rec["config"]["caches"].startswith("warm")
    assert "cpu_baseline" not in rec
    # the useful FLOPs of one step (both chunks, closed forms) over the step time give the value
    step_flops = 4 * 128 * (56 * (2048 * 6145 + 2047 * 2048 // 2) + 32 * (2048 * 30721 + 2047 * 2048 // 2))
    assert abs(rec["value"] - step_flops / (rec["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * rec["value"] + 0.01
