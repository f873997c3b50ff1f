"""CPU oracle for grouped-query prefill attention -- test infrastructure only.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use
this package. It shares no code with the HIP library under ``prefill_attention_amd/``.
"""
from .sdpa import (  # noqa: F401
    NO_CAUSAL,
    additive_mask,
    attention_rows,
    bf16_bits_to_f64,
    brute_sdpa,
    host_workers,
    kv_head_of,
    oracle_sdpa,
    oracle_selected_rows,
    visible,
    visible_pair_count,
)
from .varlen import oracle_varlen, oracle_varlen_rows, varlen_visible  # noqa: F401
