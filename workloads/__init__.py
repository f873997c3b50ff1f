"""Seeded synthetic workloads for grouped-query prefill attention.

This module is shared by the HIP path's tests and bench and by the CPU oracle. It holds no attention
arithmetic: only the table of workload shapes and mask arguments, and the generator of the bf16 input
bits that both sides consume. The GPU receives the bits through a bf16 view; the oracle widens the
same bits to fp64 by itself.

Workload recipe (shapes from the pages' workloads, values synthetic):

* Q, K, V are drawn as float32 standard normals from ``numpy.random.default_rng(seed)`` in the
  order Q, K, V, then (only for the key-padding workload) the per-sequence valid lengths.
* An amplitude factor (a power of two, so exact) scales the draws; the small prompt case uses 0.5.
* Each float32 is rounded to bf16 with round-to-nearest-even on its bit pattern.
* ``scale`` is the float32 value of ``1/sqrt(D)``, handed to both sides unchanged.
* Key padding: ``key_mask[b, j] = 1`` for ``j < n_b`` with ``n_b`` drawn uniformly from the
  integers 1024..4096 inclusive.
* Additive bias ``[L, S]``: ``2 * N(0, 1)`` float32, drawn after Q, K, V.
* Attention sinks ``[Hq]``: ``N(0, 1)`` float32 logits, drawn after Q, K, V (and the bias).
* Block bitmap ``[Hq, ceil(L/block_q), ceil(S/block_k)]`` (uint8, broadcast over the batch): the
  key block holding the query block's last causal key and key block 0 are always selected, every
  other key block with probability ``density`` (uniform draws after Q, K, V, bias and sinks) --
  a selection that keeps the local block and a few distant ones, as block-sparse prefill does.
"""
from __future__ import annotations

import numpy as np

NO_CAUSAL = -1

# name -> workload.  `causal_offset` < 0 means no causal mask (bidirectional).
CONFIGS: dict[str, dict] = {
    # tiny-llm Week 2 Day 5, Task 1: the causal GQA witness, 33 query rows over 47 keys.
    "causal_witness_33x47": dict(B=1, Hq=4, Hkv=2, D=128, L=33, S=47, causal_offset=14, window=0,
                                 amp=1.0, key_padding=None),
    # Small-model prompt prefill, L = S = 128, inputs scaled by 0.5.
    "small_prompt_128": dict(B=1, Hq=16, Hkv=8, D=128, L=128, S=128, causal_offset=0, window=0,
                             amp=0.5, key_padding=None),
    # Mid-context chunk: 2048 new rows on a 6144-key prefix, Llama-style G = 7 grouping
    # (TensorFold PR, geometry DH 128, NQ 56, G 7, KVH 8).
    "mid_ctx_8k": dict(B=1, Hq=56, Hkv=8, D=128, L=2048, S=8192, causal_offset=6144, window=0,
                       amp=1.0, key_padding=None),
    # Sliding-window chunk on a rotating cache of W - 1 + L keys (mlx-lm PR, commit text).
    "sliding_w1024_d128": dict(B=1, Hq=32, Hkv=8, D=128, L=2048, S=3071, causal_offset=1023,
                               window=1024, amp=1.0, key_padding=None),
    "sliding_w1024_d64": dict(B=1, Hq=32, Hkv=8, D=64, L=2048, S=3071, causal_offset=1023,
                              window=1024, amp=1.0, key_padding=None),
    # Long-context chunk: 2048 new rows on a 30720-key prefix.
    "long_ctx_32k": dict(B=1, Hq=32, Hkv=8, D=128, L=2048, S=32768, causal_offset=30720, window=0,
                         amp=1.0, key_padding=None),
    # Batched bidirectional prefill with per-sequence key padding (encoder-style prefill).
    "bidir_padded_b8": dict(B=8, Hq=32, Hkv=8, D=128, L=4096, S=4096, causal_offset=NO_CAUSAL,
                            window=0, amp=1.0, key_padding=(1024, 4096)),
    # The long-context chunk with logit soft-capping at 50 (the Gemma-2 attention cap; brotensor
    # attn_softcap).
    "long_ctx_32k_softcap50": dict(B=1, Hq=32, Hkv=8, D=128, L=2048, S=32768, causal_offset=30720, window=0,
                                   amp=1.0, key_padding=None, softcap=50.0),
    # The mid-context chunk with an additive FP32 bias of [L, S] broadcast over batch and heads
    # (tiny-llm Task 2's broadcastable additive mask), drawn as 2 * N(0, 1) after Q, K, V.
    "mid_ctx_8k_bias": dict(B=1, Hq=56, Hkv=8, D=128, L=2048, S=8192, causal_offset=6144, window=0,
                            amp=1.0, key_padding=None, bias="LS"),
    # The sliding-window chunk through the rotating-cache entry point: the first 1023 keys are the
    # cached history (in a 3072-slot ring, key j in slot j mod 3072), the last 2048 the chunk's own
    # keys, appended by the call (TensorFold PR: ring slot of a key row; brotensor kv_cache_append).
    "ring_w1024_l2048": dict(B=1, Hq=32, Hkv=8, D=128, L=2048, S=3071, causal_offset=1023, window=1024,
                             amp=1.0, key_padding=None, entry="ring", ring=3072),
    # Short-query chunks for the decode entry point (tiny-llm Task 2 routes one-token decode and
    # L <= 8 to a separate path; brotensor flash_attention_decode: query position valid_len - L + i).
    "decode_l1_32k": dict(B=1, Hq=32, Hkv=8, D=128, L=1, S=32768, causal_offset=32767, window=0,
                          amp=1.0, key_padding=None, entry="decode"),
    "decode_l8_8k": dict(B=1, Hq=56, Hkv=8, D=128, L=8, S=8192, causal_offset=8184, window=0,
                         amp=1.0, key_padding=None, entry="decode"),
    "decode_b8_l1_4k": dict(B=8, Hq=32, Hkv=8, D=128, L=1, S=4096, causal_offset=4095, window=0,
                            amp=1.0, key_padding=None, entry="decode"),
    # The long-context chunk with one attention-sink logit per query head (mlx-lm sliding-window
    # prefill PR: attention sinks among the cases its prefill path reproduces).
    "long_ctx_32k_sinks": dict(B=1, Hq=32, Hkv=8, D=128, L=2048, S=32768, causal_offset=30720, window=0,
                               amp=1.0, key_padding=None, sinks=True),
    # The long-context chunk under a block bitmap (TensorFold PR: MiniMax-M3's block bitmap SEL):
    # query blocks of 128 rows select 512-key blocks, about a quarter of the causal blocks.
    "long_ctx_32k_sel": dict(B=1, Hq=32, Hkv=8, D=128, L=2048, S=32768, causal_offset=30720, window=0,
                             amp=1.0, key_padding=None, block_sel=dict(block_q=128, block_k=512, density=0.25)),
    # The long-context chunk on one GPU's share of a model with 64 query and 8 KV heads split over
    # 8 GPUs by KV head: one KV head and its 8 query heads, 64 query blocks of 256 rows -- fewer than
    # the 256 compute units. Once through the one-workgroup-per-block entry point and once through
    # the key split with a caller workspace.
    "few_heads_32k": dict(B=1, Hq=8, Hkv=1, D=128, L=2048, S=32768, causal_offset=30720, window=0,
                          amp=1.0, key_padding=None),
    "few_heads_32k_split": dict(B=1, Hq=8, Hkv=1, D=128, L=2048, S=32768, causal_offset=30720, window=0,
                                amp=1.0, key_padding=None, entry="split"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even) and return the uint16 bits.

    Inputs must be finite (the generators never produce NaN or infinity)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def make_inputs(cfg: dict | str, seed: int = 0, **overrides) -> dict:
    """Draw one workload's inputs.

    Returns a dict with ``q``, ``k``, ``v`` (uint16 bf16 bit arrays of shapes [B,Hq,L,D],
    [B,Hkv,S,D], [B,Hkv,S,D]), ``key_mask`` (uint8 [B,S] or None), ``key_lengths`` (or None),
    ``scale`` (numpy float32) and the shape/mask arguments.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    c = dict(cfg)
    c.update(overrides)
    B, Hq, Hkv, D, L, S = (int(c[n]) for n in ("B", "Hq", "Hkv", "D", "L", "S"))
    amp = np.float32(c.get("amp", 1.0))
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, L, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    if amp != 1.0:
        q *= amp
        k *= amp
        v *= amp
    key_mask = None
    lengths = None
    kp = c.get("key_padding")
    if kp is not None:
        lo, hi = kp
        lengths = rng.integers(lo, hi + 1, size=B)
        key_mask = (np.arange(S)[None, :] < lengths[:, None]).astype(np.uint8)
    bias = None
    if c.get("bias") == "LS":
        bias = (rng.standard_normal((L, S), dtype=np.float32) * np.float32(2.0))
    sinks = rng.standard_normal(Hq, dtype=np.float32) if c.get("sinks") else None
    block_sel = None
    bs = c.get("block_sel")
    if bs is not None:
        bq, bk = int(bs["block_q"]), int(bs["block_k"])
        nqb, nkb = -(-L // bq), -(-S // bk)
        block_sel = (rng.random((Hq, nqb, nkb)) < float(bs["density"])).astype(np.uint8)
        block_sel[:, :, 0] = 1
        off = int(c.get("causal_offset", NO_CAUSAL))
        if off >= 0:
            for qb in range(nqb):
                last = min(S - 1, min(L, (qb + 1) * bq) - 1 + off)
                block_sel[:, qb, last // bk] = 1
    return dict(
        q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v),
        key_mask=key_mask, key_lengths=lengths, bias=bias, sinks=sinks, block_sel=block_sel,
        block_q=int(bs["block_q"]) if bs else 0, block_k=int(bs["block_k"]) if bs else 0,
        scale=np.float32(1.0 / np.sqrt(np.float32(D))) if c.get("scale") is None else np.float32(c["scale"]),
        B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, S=S,
        causal_offset=int(c.get("causal_offset", NO_CAUSAL)), window=int(c.get("window", 0)),
    )


def random_bits(rng: np.random.Generator, shape, amp: float = 1.0) -> np.ndarray:
    """bf16 bits of amp * N(0,1) float32 draws from an existing generator."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if amp != 1.0:
        x *= np.float32(amp)
    return f32_to_bf16_bits(x)


# ----------------------------------------------------------------------------------------------
# Packed variable-length batches (brotensor flash_attention_varlen_forward layout)
# ----------------------------------------------------------------------------------------------
# name -> workload. Query lengths are drawn from `lq` (inclusive range); each sequence's keys are
# its cached prefix (drawn from `prefix`, inclusive) followed by its query rows, so Lk = prefix + Lq.
VARLEN_CONFIGS: dict[str, dict] = {
    # Batched causal prompt prefill, 8 packed sequences of 1024..4096 tokens (the key-padding
    # workload's length mix, packed instead of padded), Lq == Lk.
    "varlen_causal_b8": dict(n_seq=8, Hq=32, Hkv=8, D=128, lq=(1024, 4096), prefix=(0, 0), causal=True,
                             window=0),
    # Ragged chunks after cached prefixes: short and long rows, several key tiles, ragged tails.
    "varlen_chunks_b5": dict(n_seq=5, Hq=8, Hkv=2, D=128, lq=(1, 300), prefix=(0, 500), causal=True,
                             window=0),
}


def make_varlen_inputs(cfg: dict | str, seed: int = 0, lengths_q=None, lengths_k=None, **overrides) -> dict:
    """Draw one packed variable-length workload.

    Draw order from ``numpy.random.default_rng(seed)``: the n_seq query lengths, the n_seq prefix
    lengths, then Q [total_q, Hq, D], K and V [total_k, Hkv, D] as float32 standard normals rounded
    to bf16. ``lengths_q`` / ``lengths_k`` override the drawn lengths (the draws still happen, so the
    value stream is the same). Returns bit arrays, int32 prefix sums ``cu_q`` / ``cu_k`` and the
    arguments."""
    if isinstance(cfg, str):
        cfg = VARLEN_CONFIGS[cfg]
    c = dict(cfg)
    c.update(overrides)
    n, Hq, Hkv, D = (int(c[k]) for k in ("n_seq", "Hq", "Hkv", "D"))
    rng = np.random.default_rng(seed)
    lq = rng.integers(c["lq"][0], c["lq"][1] + 1, size=n)
    pre = rng.integers(c["prefix"][0], c["prefix"][1] + 1, size=n)
    lk = lq + pre
    if lengths_q is not None:
        lq = np.asarray(lengths_q, dtype=np.int64)
    if lengths_k is not None:
        lk = np.asarray(lengths_k, dtype=np.int64)
    n = len(lq)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q = rng.standard_normal((tq, Hq, D), dtype=np.float32)
    k = rng.standard_normal((tk, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((tk, Hkv, D), dtype=np.float32)
    return dict(
        q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v),
        cu_q=cu_q, cu_k=cu_k, lengths_q=lq.astype(np.int64), lengths_k=lk.astype(np.int64),
        n_seq=n, Hq=Hq, Hkv=Hkv, D=D, total_q=tq, total_k=tk, max_seqlen_q=int(max(1, lq.max(initial=1))),
        scale=np.float32(1.0 / np.sqrt(np.float32(D))), causal=bool(c.get("causal", True)),
        window=int(c.get("window", 0)),
    )
