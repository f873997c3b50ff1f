"""Grouped-query flash prefill attention for AMD Instinct MI355X (gfx950).

The computation runs in ``libpfa.so`` (hand-written HIP); this package is its thin Python binding.
Every call takes bf16 torch tensors on one GPU, enqueues on the current stream (or ``stream=``)
and raises ``PfaError`` with the library's status on any invalid argument; there is no CPU
fallback.

- ``prefill_attn_gqa(q, k, v, ...)``: Q ``[B, Hq, L, D]`` against K, V ``[B, Hkv, S, D]`` with a
  causal offset (a chunk after ``S - L`` cached keys by default), a sliding window, a key mask,
  logit soft-cap, an additive bias, attention sinks or a block bitmap. With ``workspace=`` (a
  zero-filled uint8 tensor of ``prefill_workspace_bytes(...)`` bytes, reusable) calls with few query
  blocks (at most 192 of 256 rows) split their keys over the whole chip.
- ``prefill_attn_gqa_varlen(...)``: packed variable-length batches (``cu_seqlens`` prefix sums).
- ``prefill_attn_gqa_ring(...)``: causal or sliding-window prefill on a rotating K/V cache,
  appending the chunk's own keys first.
- ``prefill_attn_gqa_decode(...)``: short query chunks (1 <= L <= 64) against a long cache, split
  over the keys (workspace: ``decode_workspace_bytes(...)``); ``prefill_attn_gqa_decode_noalloc``
  does the same without allocating (a library-held scratch array; calls on one GPU must not
  overlap).
"""
from ._binding import (  # noqa: F401
    DECODE_MAX_L,
    DECODE_SCRATCH_BYTES,
    EXPORTS,
    FLAG_NO_SKIP,
    LIB_PATH,
    MAX_LEN,
    NO_CAUSAL,
    Options,
    STATUS,
    PfaError,
    decode_workspace_bytes,
    library,
    prefill_attn_gqa,
    prefill_attn_gqa_decode,
    prefill_attn_gqa_decode_noalloc,
    prefill_attn_gqa_decode_noalloc_raw,
    prefill_attn_gqa_decode_raw,
    prefill_attn_gqa_raw,
    prefill_attn_gqa_ws_raw,
    prefill_workspace_bytes,
    prefill_attn_gqa_ring,
    prefill_attn_gqa_ring_raw,
    prefill_attn_gqa_varlen,
    prefill_attn_gqa_varlen_raw,
    status_str,
    version,
)
