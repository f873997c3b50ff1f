"""Grouped-query flash prefill attention for AMD Instinct MI355X (gfx950).

The computation runs in ``libpfa.so`` (hand-written HIP); this package is its thin Python binding.
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
