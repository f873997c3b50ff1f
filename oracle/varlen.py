"""CPU oracle for packed variable-length grouped-query attention (fp64, explicit mask).

TEST INFRASTRUCTURE ONLY (same rules as ``oracle.sdpa``): used by the test-suite and the bench's
CPU-baseline leg, never by the product path; shares no code with the HIP library.

Definition (brotensor flash_attention.h, flash_attention_varlen_forward): all sequences live back to
back in packed tensors Q [total_q, Hq, D], K / V [total_k, Hkv, D]; sequence b owns query rows
[cu_q[b], cu_q[b+1]) and keys [cu_k[b], cu_k[b+1]); no query attends to a key of another sequence.
Within a sequence the attention is the plain masked SDPA of ``oracle.sdpa`` with grouped-query heads
(query head h reads KV head h // (Hq / Hkv)).

Causal term, per sequence: the page states it for equal query and key lengths as
``(k - cu_k[b]) <= (q - cu_q[b])``, i.e. local key j visible to local row i iff j <= i. Reading
taken for unequal lengths: the rows are the last Lq positions of the sequence's Lk keys (a chunk
after its cached prefix, the alignment of tiny-llm Week 2 Day 5 Task 2 and of the tinygrad prefill
mask), so j <= i + (Lk - Lq); this reduces to the page's rule when Lq == Lk. Window term (as in
``oracle.sdpa``): j >= i + (Lk - Lq) - W + 1 when W > 0. A row with no visible key outputs zeros.
The logit soft-cap and the attention sinks are those of ``oracle.sdpa`` (same functions).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .sdpa import _softmax_rows_times_v, _widen, kv_head_of, soft_cap


def varlen_visible(Lq: int, Lk: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [Lq, Lk]: may local row i of a sequence attend local key j."""
    i = np.arange(Lq, dtype=np.int64)[:, None]
    j = np.arange(Lk, dtype=np.int64)[None, :]
    vis = np.ones((Lq, Lk), dtype=bool)
    if causal:
        off = Lk - Lq
        vis &= j <= i + off
        if window > 0:
            vis &= j >= i + off - window + 1
    return vis


def oracle_varlen(q, k, v, cu_q, cu_k, scale, causal: bool = True, window: int = 0, softcap: float = 0.0,
                  sinks=None, workers: int = 1) -> np.ndarray:
    """Packed variable-length SDPA in fp64. q: [total_q, Hq, D], k/v: [total_k, Hkv, D] as bf16 bits
    (uint16) or floats; cu_q / cu_k: prefix sums of n_seq + 1 entries; softcap > 0: logit soft-cap;
    sinks: [Hq] sink logits or None. Returns fp64 [total_q, Hq, D]. `workers` > 1 spreads the
    (sequence, head) items over a thread pool (numpy releases the GIL)."""
    q, k, v = _widen(q), _widen(k), _widen(v)
    total_q, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if window > 0 and not causal:
        raise ValueError("a sliding window needs the causal term")
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    out = np.zeros((total_q, Hq, v.shape[-1]), dtype=np.float64)
    scale = float(np.float64(scale))
    def run(item):
        b, h = item
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        Lq, Lk = int(q1 - q0), int(k1 - k0)
        if Lq == 0 or Lk == 0:
            return  # no rows, or no keys: zeros
        add = np.where(varlen_visible(Lq, Lk, causal, window), 0.0, -np.inf)
        hk = kv_head_of(h, Hq, Hkv)
        scores = soft_cap(scale * (q[q0:q1, h] @ k[k0:k1, hk].T), float(softcap)) + add
        out[q0:q1, h] = _softmax_rows_times_v(scores, v[k0:k1, hk],
                                              None if sinks is None else float(np.float64(sinks[h])))

    items = [(b, h) for b in range(len(cu_q) - 1) for h in range(Hq)]
    if workers <= 1:
        for it in items:
            run(it)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(run, items))
    return out


def sequence_of_row(cu_q, r: int) -> int:
    """Index b of the sequence that owns packed query row r, i.e. cu_q[b] <= r < cu_q[b + 1]
    (brotensor varlen layout). A sequence without rows owns none, so among equal prefix sums the
    last one is the owner: the rightmost b with cu_q[b] <= r."""
    return int(np.searchsorted(np.asarray(cu_q, dtype=np.int64), r, side="right") - 1)


def oracle_varlen_rows(q, k, v, cu_q, cu_k, scale, causal, window, picks, softcap: float = 0.0,
                       sinks=None) -> np.ndarray:
    """Oracle output for selected (packed row, query head) pairs only: fp64 [len(picks), D]. The
    same definition as oracle_varlen, one row at a time (used at full workload sizes, where every
    row would take too long); the row's sequence comes from sequence_of_row."""
    Hq, Hkv = q.shape[1], k.shape[1]
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    res = []
    for (r, h) in picks:
        b = sequence_of_row(cu_q, r)
        q0, k0, k1 = cu_q[b], cu_k[b], cu_k[b + 1]
        Lq, Lk = int(cu_q[b + 1] - q0), int(k1 - k0)
        i = int(r - q0)
        hk = kv_head_of(h, Hq, Hkv)
        vis = varlen_visible(Lq, Lk, causal, window)[i:i + 1]
        if Lk == 0 or not vis.any():
            res.append(np.zeros(v.shape[-1]))
            continue
        kk, vv = _widen(k[k0:k1, hk]), _widen(v[k0:k1, hk])
        scores = soft_cap(float(np.float64(scale)) * (_widen(q[r:r + 1, h]) @ kk.T), float(softcap))
        scores = scores + np.where(vis, 0.0, -np.inf)
        res.append(_softmax_rows_times_v(scores, vv, None if sinks is None else float(np.float64(sinks[h])))[0])
    return np.array(res)
