"""Throughput of grouped-query flash prefill attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --calibrate-copy     (three plain 1 GiB device copies: the reference kernel
                                          that HBM byte counters are scaled against)

A step is one pass of the prefill attention over one batch of each workload chunk, with all
inputs resident in HBM before the timed region starts. The default workload is the pair of causal
D=128 chunks that the throughput target is quoted on: 2048 new rows on an 8192-key context
(Hq=56, Hkv=8) and 2048 new rows on a 32768-key context (Hq=32, Hkv=8). Prints one JSON line.

value = useful TFLOP/s = 4 * D * (visible query-key pairs) / time, whole job.
roofline: the prefill kernel against the bf16 dense MFMA peak, with its average launch duration
taken from HIP events recorded on the launch stream around every launch of the timed region.
cpu_baseline: the fp64 CPU oracle, timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attn useful TFLOP/s + % bf16 MFMA peak; query tok/s at 8K/32K ctx"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "prefill_attention_amd", "csrc", "pfa_kernel.hip")
COUNTERS_MD = os.path.join(ROOT, "profiles", "pfa_prefill_kernel_causal_8k_32k_counters.md")

WORKLOADS = {
    "causal_8k_32k": ["mid_ctx_8k", "long_ctx_32k"],
    "mid_ctx_8k": ["mid_ctx_8k"],
    "long_ctx_32k": ["long_ctx_32k"],
    "sliding_w1024_d128": ["sliding_w1024_d128"],
    "sliding_w1024_d64": ["sliding_w1024_d64"],
    "bidir_padded_b8": ["bidir_padded_b8"],
    "small_prompt_128": ["small_prompt_128"],
    "causal_witness_33x47": ["causal_witness_33x47"],
}
DESCRIPTION = {
    "causal_8k_32k": "causal GQA prefill chunks, L=2048 on S=8192 (Hq=56,Hkv=8) and on S=32768 "
                     "(Hq=32,Hkv=8), D=128, one of each per step",
}


def visible_pairs(c: dict, key_lengths=None) -> int:
    """Visible (row, key) cells over all query heads, closed form per row."""
    B, Hq, L, S = c["B"], c["Hq"], c["L"], c["S"]
    off, W = c["causal_offset"], c["window"]
    if off < 0:
        per_b = [int(n) for n in key_lengths] if key_lengths is not None else [S] * B
        return Hq * L * sum(per_b)
    total = 0
    for i in range(L):
        hi = min(S - 1, i + off)
        lo = max(0, i + off - W + 1) if W > 0 else 0
        total += max(0, hi - lo + 1)
    return B * Hq * total


def algorithmic_bytes(c: dict) -> int:
    B, Hq, Hkv, L, S, D = c["B"], c["Hq"], c["Hkv"], c["L"], c["S"], c["D"]
    mask = B * S if c.get("key_padding") else 0
    return 2 * (B * Hq * L * D + 2 * B * Hkv * S * D + B * Hq * L * D) + mask


def kernel_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel source for this workload; else None."""
    if workload != "causal_8k_32k" or not os.path.exists(COUNTERS_MD):
        return None
    text = open(COUNTERS_MD).read()
    sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not val or sha.group(1) != kernel_sha():
        return None
    return float(val.group(1))


def cpu_baseline(workers: int, budget_s: float = 20.0) -> dict:
    """The oracle as it stands, on a bounded sample of the 8K chunk: heads taken one by one (all
    2048 rows each) until about `budget_s` of wall time has passed."""
    import numpy as np

    from oracle import oracle_sdpa
    from workloads import CONFIGS, make_inputs

    c = CONFIGS["mid_ctx_8k"]
    x = make_inputs("mid_ctx_8k", seed=0)
    G = c["Hq"] // c["Hkv"]
    per_head_pairs = visible_pairs(dict(c, B=1, Hq=1))
    heads = 0
    t0 = time.perf_counter()
    step = max(1, workers // 8)
    while time.perf_counter() - t0 < budget_s and heads < c["Hq"]:
        h1 = min(c["Hq"], heads + step)
        hk0, hk1 = heads // G, (h1 - 1) // G + 1
        # the oracle maps query head h to KV head h // G; slice whole groups and keep the map
        q = x["q"][:, heads:h1]
        k = x["k"][:, hk0:hk1]
        v = x["v"][:, hk0:hk1]
        if (heads % G) != 0 or (h1 - heads) % G != 0:
            # partial group: run head by head against its own KV head
            for h in range(heads, h1):
                oracle_sdpa(x["q"][:, h:h + 1], x["k"][:, h // G:h // G + 1], x["v"][:, h // G:h // G + 1],
                            x["scale"], c["causal_offset"], c["window"], None, workers=workers)
        else:
            oracle_sdpa(q, k, v, x["scale"], c["causal_offset"], c["window"], None, workers=workers)
        heads = h1
    dt = time.perf_counter() - t0
    flops = 4.0 * c["D"] * per_head_pairs * heads
    del np
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"mid_ctx_8k (L=2048, S=8192, D=128): {heads} of {c['Hq']} query heads, all rows, "
                      f"fp64 NumPy, {dt:.1f} s wall, {workers} threads"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="causal_8k_32k", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this prefill-attention library has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import prefill_attention_amd as pfa
    from workloads import CONFIGS, make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        a = torch.ones(2 ** 28, dtype=torch.int32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print("copied 3 x 1 GiB", flush=True)
        return 0
    calls = []
    total_flops = 0
    per_cfg = []
    for name in WORKLOADS[args.workload]:
        c = CONFIGS[name]
        x = make_inputs(name, seed=0)

        def t(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

        q, k, v = t(x["q"]), t(x["k"]), t(x["v"])
        m = torch.from_numpy(x["key_mask"]).to(dev) if x["key_mask"] is not None else None
        out = torch.empty_like(q)
        causal = x["causal_offset"] >= 0
        kw = dict(scale=float(x["scale"]), causal=causal,
                  causal_offset=x["causal_offset"] if causal else None, window=x["window"],
                  key_mask=m, out=out)
        flops = 4 * c["D"] * visible_pairs(c, x["key_lengths"])
        total_flops += flops
        calls.append((name, q, k, v, kw))
        per_cfg.append(dict(name=name, flops=flops, rows=c["B"] * c["L"], bytes=algorithmic_bytes(c)))
    torch.cuda.synchronize()

    def step(events=None):
        for idx, (name, q, k, v, kw) in enumerate(calls):
            if events is not None:
                events[idx][0].record()
            pfa.prefill_attn_gqa(q, k, v, **kw)
            if events is not None:
                events[idx][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step timing
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-launch durations (HIP events on the launch stream = torch's current stream)
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in calls] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    per_launch_ms = [[ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)] for i in range(len(calls))]
    mean_ms = [float(np.mean(v)) for v in per_launch_ms]

    ms_per_step = wall * 1e3 / args.steps
    value = total_flops / (wall / args.steps) / 1e12
    kernel_ms_total = sum(mean_ms)
    achieved = total_flops / (kernel_ms_total * 1e-3) / 1e12
    traffic = recorded_traffic(args.workload)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload,
                   "description": DESCRIPTION.get(args.workload, args.workload),
                   "chunks": [CONFIGS[n] | {"name": n} for n in WORKLOADS[args.workload]]},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "per_workload": [{
            "name": pc["name"],
            "kernel_ms": round(ms, 4),
            "useful_tflops": round(pc["flops"] / (ms * 1e-3) / 1e12, 2),
            "pct_bf16_peak": round(100.0 * pc["flops"] / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "query_tok_s": round(pc["rows"] / (ms * 1e-3), 1),
            "alg_hbm_gbs": round(pc["bytes"] / (ms * 1e-3) / 1e9, 1),
        } for pc, ms in zip(per_cfg, mean_ms)],
        "roofline": {
            "bound": "mfma",
            "kernel": "pfa_prefill_kernel<%d,%s>" % (CONFIGS[WORKLOADS[args.workload][0]]["D"],
                                                     "true" if CONFIGS[WORKLOADS[args.workload][0]]["key_padding"] else "false"),
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(kernel_ms_total / len(calls), 4),
            "useful_flops_per_launch": total_flops / len(calls),
        },
    }
    if not args.no_cpu_baseline:
        from oracle import host_workers
        workers = min(16, host_workers())
        rec["cpu_baseline"] = cpu_baseline(workers, args.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
