"""Throughput of grouped-query flash prefill attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--cold-mib N]
    python bench.py --calibrate-copy     (three plain 1 GiB device copies: the reference kernel
                                          that HBM byte counters are scaled against)

A step is one pass of the prefill attention over one batch of each workload chunk, with all
inputs resident in HBM before the timed region starts. The default workload is the pair of causal
D=128 chunks that the throughput target is quoted on: 2048 new rows on an 8192-key context
(Hq=56, Hkv=8) and 2048 new rows on a 32768-key context (Hq=32, Hkv=8). Prints one JSON line.

value = useful TFLOP/s = 4 * D * (visible query-key pairs) / time, whole job.
Defaults: at least 50 timed steps and 5 warm-up steps, and at least 0.1 s of each (short launches run
more steps); explicit --steps / --warmup are taken as given.
roofline: the prefill kernel against the bf16 dense MFMA peak, with its average launch duration
taken from HIP events recorded on the launch stream around every launch of a second timed pass
(launches under a millisecond in runs of back-to-back launches between two events).
cpu_baseline: the fp64 CPU oracle, timed on a bounded sample of the same workload.
--cold-mib N: every launch reads a different copy of Q, K, V and the key mask (and writes a different
O), cycling through enough copies to exceed N MiB, so that no launch finds its operands in the L2 or
the 256 MB last-level (MALL) cache; 0 reuses the same buffers (warm). Bias, sinks and bitmaps are
shared by the copies, and the rotating-cache workload always reuses its cache. Workloads whose arithmetic
intensity is below the ridge (bf16 peak / HBM peak, about 315 flop/byte: decode, small prompts) are
HBM-bound: they default to cold (512 MiB; a one-token call on a 32K cache reads 134 MB, which the
last-level cache would otherwise serve in part) and report their roofline against HBM bandwidth with
algorithmic bytes; the others default to warm and report against the MFMA peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
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
    "varlen_causal_b8": ["varlen_causal_b8"],
    "long_ctx_32k_softcap50": ["long_ctx_32k_softcap50"],
    "mid_ctx_8k_bias": ["mid_ctx_8k_bias"],
    "ring_w1024_l2048": ["ring_w1024_l2048"],
    "decode_l1_32k": ["decode_l1_32k"],
    "decode_l8_8k": ["decode_l8_8k"],
    "decode_b8_l1_4k": ["decode_b8_l1_4k"],
    "long_ctx_32k_sinks": ["long_ctx_32k_sinks"],
    "long_ctx_32k_sel": ["long_ctx_32k_sel"],
    "few_heads_32k": ["few_heads_32k"],
    "few_heads_32k_split": ["few_heads_32k_split"],
}
DESCRIPTION = {
    "causal_8k_32k": "causal GQA prefill chunks, L=2048 on S=8192 (Hq=56,Hkv=8) and on S=32768 "
                     "(Hq=32,Hkv=8), D=128, one of each per step",
    "varlen_causal_b8": "packed variable-length causal GQA prompt prefill, 8 sequences of 1024..4096 "
                        "tokens (Lq == Lk), Hq=32, Hkv=8, D=128, one launch per step",
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


def below_ridge(workload: str) -> bool:
    """Whether the workload's useful flops per algorithmic byte fall below the bf16-MFMA / HBM ridge
    (key-padded chunks counted at full length: an upper bound on their flops)."""
    from workloads import CONFIGS

    names = [n for n in WORKLOADS[workload] if n in CONFIGS]
    if len(names) != len(WORKLOADS[workload]):
        return False  # packed varlen batches: long causal prompts, far above the ridge
    flops = sum(4 * CONFIGS[n]["D"] * visible_pairs(CONFIGS[n]) for n in names)
    return flops / sum(algorithmic_bytes(CONFIGS[n]) for n in names) < PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3


def sel_visible_pairs(c: dict, block_sel, block_q: int, block_k: int) -> int:
    """Visible (row, key) cells over all query heads under a causal mask and a block bitmap
    [Hq, n_qblocks, n_kblocks]: per row, the causal key range [0, i + off] intersected with the
    selected key blocks, counted block by block."""
    import numpy as np

    L, S, off = c["L"], c["S"], c["causal_offset"]
    i = np.arange(L, dtype=np.int64)
    hi = np.minimum(S - 1, i + off) if off >= 0 else np.full(L, S - 1, dtype=np.int64)  # last visible key
    nkb = block_sel.shape[2]
    kb0 = np.arange(nkb, dtype=np.int64) * block_k
    # keys of block kb visible to row i: clamp(hi_i + 1 - kb0, 0, min(block_k, S - kb0))
    width = np.minimum(block_k, S - kb0)
    per = np.clip(hi[:, None] + 1 - kb0[None, :], 0, width[None, :])  # [L, nkb]
    qb = i // block_q
    total = 0
    for h in range(block_sel.shape[0]):
        total += int((per * block_sel[h][qb]).sum())
    return c["B"] * total


def varlen_visible_pairs(x: dict) -> int:
    """Visible (row, key) cells over all query heads of a packed batch, closed form per row."""
    import numpy as np

    total = 0
    for lq, lk in zip(x["lengths_q"], x["lengths_k"]):
        i = np.arange(int(lq), dtype=np.int64)
        if x["causal"]:
            off = int(lk) - int(lq)
            hi = np.minimum(int(lk) - 1, i + off)
            lo = np.maximum(0, i + off - x["window"] + 1) if x["window"] > 0 else np.zeros_like(i)
        else:
            hi = np.full_like(i, int(lk) - 1)
            lo = np.zeros_like(i)
        total += int(np.maximum(0, hi - lo + 1).sum())
    return total * x["Hq"]


def varlen_algorithmic_bytes(x: dict) -> int:
    D = x["D"]
    return 2 * (2 * x["total_q"] * x["Hq"] * D + 2 * x["total_k"] * x["Hkv"] * D) + 8 * (x["n_seq"] + 1)


def algorithmic_bytes(c: dict) -> int:
    B, Hq, Hkv, L, S, D = c["B"], c["Hq"], c["Hkv"], c["L"], c["S"], c["D"]
    mask = B * S if c.get("key_padding") else 0
    bias = 4 * L * S if c.get("bias") == "LS" else 0
    return 2 * (B * Hq * L * D + 2 * B * Hkv * S * D + B * Hq * L * D) + mask + bias


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


def cgroup_cpu_quota():
    """Whole cores granted by the cgroup CPU quota (cgroup v2 cpu.max or v1 cfs files), or None."""
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            return max(1, int(int(quota) // int(period)))
        return None
    except (OSError, ValueError):
        pass
    try:
        with open("/sys/fs/cgroup/cpu/cpu.cfs_quota_us") as f:
            quota = int(f.read())
        with open("/sys/fs/cgroup/cpu/cpu.cfs_period_us") as f:
            period = int(f.read())
        return max(1, quota // period) if quota > 0 else None
    except (OSError, ValueError):
        return None


def blas_single_thread():
    """Context that pins the BLAS library to one thread per calling thread, so that `cores` is the
    number of worker threads actually used."""
    from threadpoolctl import threadpool_limits

    return threadpool_limits(limits=1, user_api="blas")


def cpu_baseline(workload: str, workers: int, budget_s: float = 20.0) -> dict:
    """The oracle as it stands, on a bounded sample of the workload: its chunks in order, one
    (batch element, KV group) at a time -- the group's query heads, all their rows, with the
    workload's masks and options -- until about `budget_s` of oracle time has passed or the whole
    workload is done. Useful FLOPs of the sample come from the oracle's own visible-pair count
    (outside the timed calls); the oracle itself computes every row against all S keys, so its
    dense rate is reported in the sample text as well."""
    from oracle import oracle_sdpa, visible_pair_count
    from workloads import CONFIGS, make_inputs

    done = []
    total_flops = dense_flops = 0.0
    spent = 0.0
    limit = blas_single_thread()
    limit.__enter__()
    for name in WORKLOADS[workload]:
        c = CONFIGS[name]
        x = make_inputs(name, seed=0)
        B, Hq, Hkv, L, S, D = c["B"], c["Hq"], c["Hkv"], c["L"], c["S"], c["D"]
        G = Hq // Hkv
        units = 0
        for b in range(B):
            for hk in range(Hkv):
                if spent >= budget_s:
                    break
                hs = slice(hk * G, (hk + 1) * G)
                km = x["key_mask"][b:b + 1] if x["key_mask"] is not None else None
                sel = x["block_sel"][hs] if x.get("block_sel") is not None else None
                t0 = time.perf_counter()
                oracle_sdpa(x["q"][b:b + 1, hs], x["k"][b:b + 1, hk:hk + 1], x["v"][b:b + 1, hk:hk + 1], x["scale"],
                            x["causal_offset"], x["window"], km, workers=workers,
                            softcap=float(c.get("softcap") or 0.0), bias=x.get("bias"),
                            sinks=x["sinks"][hs] if x.get("sinks") is not None else None,
                            block_sel=sel, block_q=x.get("block_q") or 0, block_k=x.get("block_k") or 0)
                spent += time.perf_counter() - t0
                units += 1
                total_flops += 4.0 * D * visible_pair_count(1, G, L, S, x["causal_offset"], x["window"], km,
                                                             block_sel=sel, block_q=x.get("block_q") or 0,
                                                             block_k=x.get("block_k") or 0)
                dense_flops += 4.0 * D * G * L * S
        done.append(f"{name} {units}/{B * Hkv} (batch element, KV group) units")
    limit.__exit__(None, None, None)
    return {"value": total_flops / spent / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{workload}, all rows of each unit's query heads (one KV group): {', '.join(done)}; fp64 NumPy, "
                      f"{spent:.1f} s in the oracle, {workers} threads x 1 BLAS thread; counting the dense "
                      f"L x S work it does, {dense_flops / spent / 1e12:.3f} TFLOP/s"}


def kernel_name(workload_name: str) -> str:
    """Name of the dominant kernel as rocprofv3 prints it (prefill MODE bits: 1 key mask, 2 ring,
    4 soft-cap, 8 bias, 16 block bitmap; the last argument is true for the key split)."""
    from workloads import CONFIGS, VARLEN_CONFIGS

    if workload_name in VARLEN_CONFIGS:
        return "pfa_prefill_kernel<%d, 0, false>" % VARLEN_CONFIGS[workload_name]["D"]
    c = CONFIGS[workload_name]
    if c.get("entry") == "decode":
        rows = (c["Hq"] // c["Hkv"]) * c["L"]
        sc = "true" if c.get("softcap") else "false"
        # up to 64 rows per KV head in 32-row groups (the register-K kernel without a key mask),
        # more in 64-row groups
        if rows <= 64 and not c["key_padding"]:
            split = "pfa_decode_kreg_kernel<%d, %s>" % (c["D"], sc)
        else:
            split = "pfa_decode_split_kernel<%d, %d, %s, %s>" % (
                c["D"], 2 if rows > 64 else 1, "true" if c["key_padding"] else "false", sc)
        return "%s + pfa_decode_merge_kernel<%d>" % (split, c["D"])
    mode = (1 if c["key_padding"] else 0) | (2 if c.get("entry") == "ring" else 0) | \
        (4 if c.get("softcap") else 0) | (8 if c.get("bias") else 0) | (16 if c.get("block_sel") else 0)
    suffix = " (after pfa_ring_append_kernel)" if c.get("entry") == "ring" else ""
    split = "true" if c.get("entry") == "split" else "false"
    return "pfa_prefill_kernel<%d, %d, %s>%s" % (c["D"], mode, split, suffix)


def varlen_cpu_baseline(name: str, workers: int, budget_s: float = 20.0) -> dict:
    """The varlen oracle as it stands, on a bounded sample of the packed workload: the first
    sequence alone, its query heads one by one, until about `budget_s` of wall time has passed."""
    import numpy as np

    from oracle import oracle_varlen
    from workloads import make_varlen_inputs

    x = make_varlen_inputs(name, seed=0)
    s0, s1 = int(x["cu_q"][0]), int(x["cu_q"][1])
    k0, k1 = int(x["cu_k"][0]), int(x["cu_k"][1])
    G = x["Hq"] // x["Hkv"]
    one = dict(x, lengths_q=x["lengths_q"][:1], lengths_k=x["lengths_k"][:1], Hq=1)
    per_head_flops = 4 * x["D"] * varlen_visible_pairs(one)
    cu_q = np.array([0, s1 - s0], dtype=np.int32)
    cu_k = np.array([0, k1 - k0], dtype=np.int32)
    from concurrent.futures import ThreadPoolExecutor

    def one_head(h):
        oracle_varlen(x["q"][s0:s1, h:h + 1], x["k"][k0:k1, h // G:h // G + 1], x["v"][k0:k1, h // G:h // G + 1],
                      cu_q, cu_k, x["scale"], x["causal"], x["window"])

    heads = 0
    t0 = time.perf_counter()
    with blas_single_thread(), ThreadPoolExecutor(max_workers=workers) as ex:
        while time.perf_counter() - t0 < budget_s and heads < x["Hq"]:
            h1 = min(x["Hq"], heads + workers)
            list(ex.map(one_head, range(heads, h1)))
            heads = h1
    dt = time.perf_counter() - t0
    return {"value": per_head_flops * heads / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{name}: sequence 0 (Lq={s1 - s0}, Lk={k1 - k0}), {heads} of {x['Hq']} query heads, "
                      f"fp64 NumPy, {dt:.1f} s wall, {workers} threads x 1 BLAS thread"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # default K / W: at least 50 timed steps and 5 warm-up steps, and at least 0.1 s of timed work and
    # of warm-up (a short launch, such as a decode call of 25 us, then runs a few thousand steps, so
    # the clock has settled and the timed region is not a few milliseconds long)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="causal_8k_32k", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--cold-mib", type=int, default=None)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this prefill-attention library has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import prefill_attention_amd as pfa
    from workloads import CONFIGS, VARLEN_CONFIGS, make_inputs, make_varlen_inputs

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
    cold_copies = {}
    if args.cold_mib is None:
        args.cold_mib = 512 if below_ridge(args.workload) else 0
    def t(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    for name in WORKLOADS[args.workload]:
        if name in VARLEN_CONFIGS:
            x = make_varlen_inputs(name, seed=0)
            q, k, v = t(x["q"]), t(x["k"]), t(x["v"])
            kw = dict(scale=float(x["scale"]), causal=x["causal"], window=x["window"], out=torch.empty_like(q))
            cq = torch.from_numpy(x["cu_q"]).to(dev)
            ck = torch.from_numpy(x["cu_k"]).to(dev)
            mq = x["max_seqlen_q"]

            def launch(q=q, k=k, v=v, cq=cq, ck=ck, mq=mq, kw=kw):
                pfa.prefill_attn_gqa_varlen(q, k, v, cq, ck, mq, **kw)

            flops = 4 * x["D"] * varlen_visible_pairs(x)
            total_flops += flops
            calls.append((name, launch))
            per_cfg.append(dict(name=name, flops=flops, rows=x["total_q"], bytes=varlen_algorithmic_bytes(x)))
            continue
        c = CONFIGS[name]
        x = make_inputs(name, seed=0)

        q, k, v = t(x["q"]), t(x["k"]), t(x["v"])
        m = torch.from_numpy(x["key_mask"]).to(dev) if x["key_mask"] is not None else None
        out = torch.empty_like(q)
        causal = x["causal_offset"] >= 0
        kw = dict(scale=float(x["scale"]), causal=causal,
                  causal_offset=x["causal_offset"] if causal else None, window=x["window"],
                  key_mask=m, out=out)
        if c.get("softcap"):
            kw["softcap"] = float(c["softcap"])
        if x.get("bias") is not None:
            kw["bias"] = torch.from_numpy(x["bias"]).to(dev)
        if x.get("sinks") is not None:
            kw["sinks"] = torch.from_numpy(x["sinks"]).to(dev)
        if x.get("block_sel") is not None:
            kw.update(block_sel=torch.from_numpy(x["block_sel"]).to(dev), block_q=x["block_q"], block_k=x["block_k"])
        if c.get("entry") == "decode":
            kw["workspace"] = torch.empty(pfa.decode_workspace_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["S"], c["D"]),
                                          dtype=torch.uint8, device=dev)
        if c.get("entry") == "split":
            # zero-filled once: the key split leaves its counters zero after every call
            kw["workspace"] = torch.zeros(pfa.prefill_workspace_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["S"], c["D"]),
                                          dtype=torch.uint8, device=dev)
        if x.get("block_sel") is not None:
            flops = 4 * c["D"] * sel_visible_pairs(c, x["block_sel"], x["block_q"], x["block_k"])
        else:
            flops = 4 * c["D"] * visible_pairs(c, x["key_lengths"])
        total_flops += flops

        fn = pfa.prefill_attn_gqa_decode if c.get("entry") == "decode" else pfa.prefill_attn_gqa

        def launch(q=q, k=k, v=v, kw=kw, fn=fn):
            fn(q, k, v, **kw)

        if args.cold_mib > 0 and c.get("entry") != "ring":
            # rotating copies: one (q, k, v, out, key mask) set per launch, cycled
            per_copy = (q.numel() + k.numel() + v.numel() + out.numel()) * 2 + (m.numel() if m is not None else 0)
            n_copies = max(2, -(-args.cold_mib * 2 ** 20 // per_copy))
            sets = [(q, k, v, out, m)] + [(q.clone(), k.clone(), v.clone(), torch.empty_like(out),
                                          m.clone() if m is not None else None) for _ in range(n_copies - 1)]
            turn = [0]

            def launch(sets=sets, kw=kw, fn=fn, turn=turn):
                qq, kk, vv, oo, mm = sets[turn[0]]
                turn[0] = (turn[0] + 1) % len(sets)
                fn(qq, kk, vv, **(kw | dict(out=oo, key_mask=mm)))

            cold_copies[name] = n_copies

        if c.get("entry") == "ring":
            pos0, ring = c["causal_offset"], c["ring"]
            k_new, v_new = k[:, :, pos0:].contiguous(), v[:, :, pos0:].contiguous()
            k_ring = torch.zeros(c["B"], c["Hkv"], ring, c["D"], dtype=torch.bfloat16, device=dev)
            v_ring = torch.zeros_like(k_ring)
            for p0 in range(max(0, pos0 - ring), pos0):
                k_ring[:, :, p0 % ring] = k[:, :, p0]
                v_ring[:, :, p0 % ring] = v[:, :, p0]

            def launch(q=q, k_new=k_new, v_new=v_new, k_ring=k_ring, v_ring=v_ring, pos0=pos0, c=c, out=out):
                pfa.prefill_attn_gqa_ring(q, k_new, v_new, k_ring, v_ring, pos0, scale=float(x["scale"]),
                                          window=c["window"], out=out)

        calls.append((name, launch))
        per_cfg.append(dict(name=name, flops=flops, rows=c["B"] * c["L"], bytes=algorithmic_bytes(c)))
    torch.cuda.synchronize()

    def step():
        for name, launch in calls:
            launch()

    # warm-up: the given number of steps, or (default) at least 5 steps and 0.1 s; the default step
    # count then comes from the warm-up's second half (past the first, slower calls)
    t0 = time.perf_counter()
    done, t_half, n_half = 0, None, 0
    while (done < args.warmup) if args.warmup is not None else (done < 5 or time.perf_counter() - t0 < 0.1):
        step()
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
            if t_half is None and time.perf_counter() - t0 >= 0.05:
                t_half, n_half = time.perf_counter(), done
    torch.cuda.synchronize()
    if t_half is not None and done > n_half:
        est = (time.perf_counter() - t_half) / (done - n_half)
    else:
        est = (time.perf_counter() - t0) / max(done, 1)
    args.warmup = done
    if args.steps is None:
        args.steps = max(50, min(5000, math.ceil(0.1 / max(est, 1e-6)))) if done > 0 else 50

    # whole-step timing
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-launch durations (HIP events on the launch stream = torch's current stream). A launch
    # shorter than a millisecond is timed in runs of `rep` back-to-back launches between two events,
    # so that the event records between launches do not add their dispatch gaps to it.
    rep = max(1, math.ceil(1e-3 / (wall / args.steps)))
    rounds = max(5, math.ceil(args.steps / rep))
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in calls] for _ in range(rounds)]
    torch.cuda.synchronize()
    for s in range(rounds):
        for idx, (name, launch) in enumerate(calls):
            ev[s][idx][0].record()
            for _ in range(rep):
                launch()
            ev[s][idx][1].record()
    torch.cuda.synchronize()
    per_launch_ms = [[ev[s][i][0].elapsed_time(ev[s][i][1]) / rep for s in range(rounds)] for i in range(len(calls))]
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
                   "caches": (f"cold: each launch reads one of {cold_copies} copies of its inputs "
                              f"(> {args.cold_mib} MiB per chunk)") if cold_copies else "warm: inputs reused",
                   "chunks": [(CONFIGS.get(n) or VARLEN_CONFIGS[n]) | {"name": n} for n in WORKLOADS[args.workload]]},
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
            "kernel": kernel_name(WORKLOADS[args.workload][0]),
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(kernel_ms_total / len(calls), 4),
            "useful_flops_per_launch": total_flops / len(calls),
        },
    }
    intensity = total_flops / sum(pc["bytes"] for pc in per_cfg)
    if intensity < PEAK_BF16_TFLOPS / PEAK_HBM_GBS * 1e3:
        # below the ridge (short queries: decode, small prompts): bound by HBM. A decode call's
        # launch time covers both of its kernels (split and merge).
        alg_bytes = sum(pc["bytes"] for pc in per_cfg) / len(calls)
        gbs = alg_bytes / (kernel_ms_total / len(calls) * 1e-3) / 1e9
        rec["roofline"] = {
            "bound": "hbm",
            "kernel": kernel_name(WORKLOADS[args.workload][0]),
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": None,
            "avg_launch_ms": round(kernel_ms_total / len(calls), 4),
            "algorithmic_bytes_per_launch": alg_bytes,
        }
    if not args.no_cpu_baseline:
        from oracle import host_workers
        affinity = host_workers()
        quota = cgroup_cpu_quota()
        # one oracle thread per core this process may actually run on: the affinity mask, bounded by
        # the cgroup CPU quota when one is set (threads beyond the quota only time-share it)
        workers = max(1, min(affinity, quota)) if quota else affinity
        if args.workload == "varlen_causal_b8":
            rec["cpu_baseline"] = varlen_cpu_baseline(args.workload, workers, args.cpu_budget)
        else:
            rec["cpu_baseline"] = cpu_baseline(args.workload, workers, args.cpu_budget)
        rec["cpu_baseline"]["affinity_cores"] = affinity
        rec["cpu_baseline"]["cpu_quota_cores"] = quota
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
