"""Host-side accounting of bench.py (CPU only): the useful-FLOP and byte counts it reports, the
cache mode it picks, its refusal of more than one GPU, and its CPU-oracle baseline on a tiny case.

The expected counts are closed forms written out here, not the bench's own row loop: a causal row i
with prefix offset `off` sees keys 0..i+off (clipped to S), a sliding-window row sees exactly W keys
once off >= W - 1, and algorithmic bytes are Q, K, V and O read or written once in bf16 (K and V
counted per KV head, never expanded to the query heads).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import CONFIGS  # noqa: E402


def causal_pairs_per_head(L, S, off):
    # rows with i + off < S see i + off + 1 keys, the rest see all S
    full = max(0, min(L, S - off))
    return full * (off + 1) + full * (full - 1) // 2 + (L - full) * S


@pytest.mark.parametrize("name, expected", [
    ("causal_witness_33x47", 4 * causal_pairs_per_head(33, 47, 14)),          # 4,092
    ("small_prompt_128", 16 * causal_pairs_per_head(128, 128, 0)),            # 132,096
    ("mid_ctx_8k", 56 * (2048 * 6145 + 2047 * 2048 // 2)),                    # 822,140,928
    ("long_ctx_32k", 32 * (2048 * 30721 + 2047 * 2048 // 2)),                 # 2,080,407,552
    ("sliding_w1024_d128", 32 * 2048 * 1024),                                 # 67,108,864
    ("sliding_w1024_d64", 32 * 2048 * 1024),
])
def test_visible_pairs_closed_form(name, expected):
    assert causal_pairs_per_head(33, 47, 14) == 1023
    assert bench.visible_pairs(CONFIGS[name]) == expected


def test_visible_pairs_key_padding():
    # bidirectional with key padding: every row of every head sees its sequence's n_b valid keys
    c = CONFIGS["bidir_padded_b8"]
    lengths = [1024, 4096, 2000, 3000, 1500, 2500, 3500, 1234]
    assert bench.visible_pairs(c, lengths) == c["Hq"] * c["L"] * sum(lengths)


@pytest.mark.parametrize("name", ["causal_witness_33x47", "small_prompt_128", "mid_ctx_8k",
                                  "sliding_w1024_d128", "sliding_w1024_d64", "long_ctx_32k", "decode_l1_32k"])
def test_algorithmic_bytes(name):
    c = CONFIGS[name]
    q = c["B"] * c["Hq"] * c["L"] * c["D"]
    kv = c["B"] * c["Hkv"] * c["S"] * c["D"]
    assert bench.algorithmic_bytes(c) == 2 * (2 * q + 2 * kv)


def test_algorithmic_bytes_values():
    assert bench.algorithmic_bytes(CONFIGS["causal_witness_33x47"]) == 115_712
    assert bench.algorithmic_bytes(CONFIGS["mid_ctx_8k"]) == 92_274_688
    assert bench.algorithmic_bytes(CONFIGS["long_ctx_32k"]) == 167_772_160
    # the key-padding mask adds one byte per key of each batch element
    c = CONFIGS["bidir_padded_b8"]
    assert bench.algorithmic_bytes(c) == 2 * (2 * 8 * 32 * 4096 * 128 + 2 * 8 * 8 * 4096 * 128) + 8 * 4096


def test_ridge_classification():
    # bf16 peak / HBM peak is about 315 flop/byte: the short-query shapes fall below it (HBM roofline,
    # cold caches by default), the long chunks far above it
    assert abs(bench.PEAK_BF16_TFLOPS / bench.PEAK_HBM_GBS * 1e3 - 314.6) < 0.1
    for name in ("causal_witness_33x47", "small_prompt_128", "decode_l1_32k", "decode_l8_8k", "decode_b8_l1_4k"):
        assert bench.below_ridge(name), name
    for name in ("causal_8k_32k", "mid_ctx_8k", "long_ctx_32k", "sliding_w1024_d128", "bidir_padded_b8",
                 "varlen_causal_b8", "ring_w1024_l2048"):
        assert not bench.below_ridge(name), name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_tiny_workload():
    r = bench.cpu_baseline("causal_witness_33x47", workers=1, budget_s=10.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["cores"] == 1
    assert r["value"] > 0
    assert "causal_witness_33x47 2/2" in r["sample"]
