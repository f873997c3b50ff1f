"""CPU oracle for grouped-query prefill attention (fp64, explicit mask).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this module; it is
used by the test-suite, by ``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``.
It shares no code with the HIP library: it reads the same seeded bf16 input bits, widens them to
fp64 itself and computes the plain definition of masked scaled-dot-product attention. The online
(streaming) softmax of the tiled method is an exact reformulation of that definition (tiny-llm,
Week 2 Day 5 "Tiled Dense Prefill Attention", Task 1, the merge equations), so the oracle is the
definition written out, not a replay of the tiles.

Definition implemented (one batch element b, one query head h):

* KV head: ``hk = floor(h / (Hq / Hkv))`` -- tiny-llm Week 2 Day 5, Task 1 (layout contract).
* Visibility of key j for query row i (``vis``), every term optional:
    - causal, aligned to the end of the cached prefix: ``j <= i + causal_offset``
      (tinygrad "symbolic llm with prefill": the prefill mask is the lower-right triangle
      ``full(-inf).triu(start_pos + 1)``; tiny-llm Task 2: row i sees through ``S - L + i``);
    - sliding window of W keys including the row's own position:
      ``j >= i + causal_offset - W + 1`` (TensorFold PR "What changes": the mask term
      ``col < row - WINDOW + 1``; brotensor ``flash_attention_windowed_forward``: keys
      ``[max(0, pos - window + 1), pos]``, window <= 0 unbounded);
    - key padding: ``key_mask[b, j] != 0`` (brotensor ``flash_attention_gqa_forward``: a
      length-Lk key mask, valid / invalid);
    - always ``j < S``.
* ``A[i, j] = 0`` if vis else ``-inf``; ``scores = scale * Q K^T + A``;
  ``O[i] = softmax(scores[i]) V``.
* Optional logit soft-capping (brotensor ``flash_attention_decode``, ``attn_softcap``: after the
  scale and before the mask and the softmax, each score ``s`` becomes ``cap * tanh(s / cap)``):
  ``scores = cap * tanh(scale * Q K^T / cap) + A`` when ``softcap = cap > 0``.
* Optional additive bias (tiny-llm Task 2: a broadcastable additive array mask, applied before the
  online-softmax update): ``scores = [soft-capped] scale * Q K^T + bias[b, h] + A``, ``bias``
  broadcastable to ``[B, Hq, L, S]``.
* Optional attention sinks (mlx-lm sliding-window prefill PR, "Correctness": attention sinks are
  among the cases its banded path must reproduce; the pages give no formula). Reading taken: one
  logit ``sink[h]`` per query head joins every row's softmax as an extra term with no value, i.e.
  ``O[i] = sum_j e^(s_ij - m) V_j / (sum_j e^(s_ij - m) + e^(sink[h] - m))`` with
  ``m = max(max_j s_ij, sink[h])``; the sink logit is used as given (not scaled, capped or biased).
* Optional block bitmap (TensorFold PR, "What changes": MiniMax-M3's kernel adds a block bitmap
  (SEL) to the masked prompt attention; the pages give no layout). Reading taken: with query blocks
  of ``block_q`` rows and key blocks of ``block_k`` keys, key j is visible to row i only if
  ``sel[b, h, i // block_q, j // block_k] != 0``, on top of every other term.
* A row with no visible key has no probability mass and its output is all zeros
  (tiny-llm Task 2), with or without a sink.

Readings taken where the pages leave a step open: ``causal_offset < 0`` means no causal term;
a window needs the causal term; the key mask is ``uint8`` with nonzero meaning valid.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

NO_CAUSAL = -1


# ----------------------------------------------------------------------------------------------
# Input widening (bf16 bits -> exact fp64)
# ----------------------------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp64 exactly: a bf16 is the top half of a float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# Head map and mask (kept as separate functions so the tests can plant mistakes in them)
# ----------------------------------------------------------------------------------------------
def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Query head h reads KV head floor(h / (Hq / Hkv)) (tiny-llm Week 2 Day 5, Task 1)."""
    group = Hq // Hkv
    return h // group


def visible(rows: np.ndarray, S: int, causal_offset: int, window: int,
            key_valid: np.ndarray | None) -> np.ndarray:
    """Boolean [len(rows), S]: may query row i attend key j.

    Causal term (lower-right): j <= i + causal_offset, applied when causal_offset >= 0
    (tinygrad prefill mask; tiny-llm Task 2). Window term: j >= i + causal_offset - window + 1
    when window > 0 (TensorFold mask term; brotensor windowed forward). Key term:
    key_valid[j] (brotensor key mask)."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(S, dtype=np.int64)[None, :]
    vis = np.ones((i.shape[0], S), dtype=bool)
    if causal_offset >= 0:
        vis &= j <= i + causal_offset
        if window > 0:
            vis &= j >= i + causal_offset - window + 1
    if key_valid is not None:
        vis &= np.asarray(key_valid, dtype=bool)[None, :]
    return vis


def block_selected(rows: np.ndarray, S: int, sel_bh: np.ndarray, block_q: int, block_k: int) -> np.ndarray:
    """Boolean [len(rows), S] from one (b, h) block bitmap sel_bh [n_qblocks, n_kblocks]: key j is
    selected for row i iff sel_bh[i // block_q, j // block_k] != 0 (TensorFold PR, SEL)."""
    qb = np.asarray(rows, dtype=np.int64) // int(block_q)
    kb = np.arange(S, dtype=np.int64) // int(block_k)
    return np.asarray(sel_bh)[qb][:, kb] != 0


def additive_mask(rows: np.ndarray, S: int, causal_offset: int, window: int,
                  key_valid: np.ndarray | None) -> np.ndarray:
    """The explicit additive mask: 0 where visible, -inf elsewhere (fp64)."""
    vis = visible(rows, S, causal_offset, window, key_valid)
    return np.where(vis, 0.0, -np.inf)


def check_args(B, Hq, Hkv, L, S, D, causal_offset, window):
    if min(B, Hq, Hkv, L, S, D) < 1:
        raise ValueError("all sizes must be >= 1")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if window > 0 and causal_offset < 0:
        raise ValueError("a sliding window needs the causal term")


# ----------------------------------------------------------------------------------------------
# The oracle proper
# ----------------------------------------------------------------------------------------------
def _softmax_rows_times_v(scores: np.ndarray, v: np.ndarray, sink: float | None = None) -> np.ndarray:
    """Plain softmax over each row of `scores` (with -inf entries), times v. Empty rows -> 0.

    With a sink logit, the softmax of each row has one more entry, `sink`, whose value is zero:
    it only adds e^(sink - m) to the normaliser."""
    m = np.max(scores, axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    if sink is not None:
        m = np.maximum(m, float(sink))
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(scores - m)          # exp(-inf) = 0 exactly
    l = np.sum(p, axis=1, keepdims=True)
    if sink is not None:
        l = l + np.exp(float(sink) - m)
    out = (p @ v) / np.where(l > 0, l, 1.0)
    out[empty] = 0.0
    return out


def soft_cap(scores: np.ndarray, softcap: float) -> np.ndarray:
    """cap * tanh(scores / cap) for cap > 0 (brotensor attn_softcap); identity for cap == 0."""
    if softcap > 0.0:
        return softcap * np.tanh(scores / softcap)
    return scores


def attention_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray,
                   scale: float, causal_offset: int, window: int,
                   key_valid: np.ndarray | None, softcap: float = 0.0,
                   bias_rows: np.ndarray | None = None, sink: float | None = None,
                   sel_rows: np.ndarray | None = None) -> np.ndarray:
    """Output rows for one (b, h): q_rows [n, D] at query positions `rows`, k/v [S, D] (fp64);
    bias_rows: the additive bias of these rows, [n, S], or None; sink: the head's sink logit or
    None; sel_rows: boolean [n, S] block selection of these rows (block_selected) or None."""
    S = k.shape[0]
    scores = soft_cap(float(scale) * (q_rows @ k.T), float(softcap))
    if bias_rows is not None:
        scores = scores + bias_rows
    scores = scores + additive_mask(rows, S, causal_offset, window, key_valid)
    if sel_rows is not None:
        scores = np.where(sel_rows, scores, -np.inf)
    return _softmax_rows_times_v(scores, v, sink)


def _widen(x):
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float64)


def oracle_sdpa(q, k, v, scale, causal_offset: int = NO_CAUSAL, window: int = 0,
                key_mask: np.ndarray | None = None, row_block: int = 256,
                workers: int = 1, softcap: float = 0.0, bias: np.ndarray | None = None,
                sinks: np.ndarray | None = None, block_sel: np.ndarray | None = None,
                block_q: int = 0, block_k: int = 0) -> np.ndarray:
    """Masked grouped-query SDPA in fp64.

    q: [B,Hq,L,D], k/v: [B,Hkv,S,D] as bf16 bits (uint16) or floats; key_mask: uint8 [B,S] or
    None; sinks: [Hq] sink logits or None; block_sel: a bitmap broadcastable to
    [B, Hq, ceil(L/block_q), ceil(S/block_k)] or None. Returns fp64 [B,Hq,L,D]. Rows are processed
    in blocks of `row_block` to bound memory; `workers` > 1 spreads (b, h, row block) items over a
    thread pool (numpy releases the GIL)."""
    q, k, v = _widen(q), _widen(k), _widen(v)
    B, Hq, L, D = q.shape
    _, Hkv, S, _ = k.shape
    check_args(B, Hq, Hkv, L, S, D, causal_offset, window)
    out = np.zeros((B, Hq, L, v.shape[-1]), dtype=np.float64)
    scale = float(np.float64(scale))
    items = [(b, h, r0) for b in range(B) for h in range(Hq) for r0 in range(0, L, row_block)]
    if bias is not None:
        bias = np.broadcast_to(np.asarray(bias, dtype=np.float64), (B, Hq, L, S))
    if block_sel is not None:
        block_sel = np.broadcast_to(np.asarray(block_sel), (B, Hq, -(-L // block_q), -(-S // block_k)))

    def run(item):
        b, h, r0 = item
        hk = kv_head_of(h, Hq, Hkv)
        rows = np.arange(r0, min(r0 + row_block, L))
        kv = None if key_mask is None else (key_mask[b] != 0)
        out[b, h, rows] = attention_rows(
            q[b, h, rows], k[b, hk], v[b, hk], rows, scale, causal_offset, window, kv, softcap,
            None if bias is None else bias[b, h, rows],
            None if sinks is None else float(np.float64(sinks[h])),
            None if block_sel is None else block_selected(rows, S, block_sel[b, h], block_q, block_k))

    if workers <= 1:
        for it in items:
            run(it)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(run, items))
    return out


def key_valid_of(key_mask: np.ndarray | None, b: int) -> np.ndarray | None:
    """The key-padding row of batch element b (brotensor key mask: nonzero = valid), or None."""
    return None if key_mask is None else (np.asarray(key_mask)[b] != 0)


def bias_of_row(bias: np.ndarray, shape: tuple, b: int, h: int, i: int) -> np.ndarray:
    """fp64 [1, S]: the additive bias of query row i of (b, h), with `bias` broadcast (numpy rules)
    to shape = (B, Hq, L, S) (tiny-llm Task 2: the additive mask broadcasts over batch and heads)."""
    full = np.broadcast_to(np.asarray(bias, dtype=np.float64), shape)
    return full[b, h, i:i + 1]


def sel_of_row(block_sel: np.ndarray, shape: tuple, block_q: int, block_k: int, b: int, h: int,
               i: int) -> np.ndarray:
    """Boolean [1, S]: the block-bitmap selection of query row i of (b, h), with `block_sel`
    broadcast to (B, Hq, ceil(L / block_q), ceil(S / block_k)); shape = (B, Hq, L, S)."""
    B, Hq, L, S = shape
    full = np.broadcast_to(np.asarray(block_sel), (B, Hq, -(-L // block_q), -(-S // block_k)))
    return block_selected(np.array([i]), S, full[b, h], block_q, block_k)


def oracle_selected_rows(q, k, v, scale, causal_offset, window, key_mask, picks,
                         softcap: float = 0.0, bias: np.ndarray | None = None,
                         sinks: np.ndarray | None = None, block_sel: np.ndarray | None = None,
                         block_q: int = 0, block_k: int = 0) -> np.ndarray:
    """Oracle output for selected (b, h, row) triples only: returns fp64 [len(picks), D].

    The same definition as oracle_sdpa, one row at a time (used at full workload sizes, where
    computing every row would take too long); each option is looked up for the picked row by
    key_valid_of, bias_of_row and sel_of_row."""
    B, Hq, L = q.shape[0], q.shape[1], q.shape[2]
    Hkv, S = k.shape[1], k.shape[2]
    shape = (B, Hq, L, S)
    res = []
    for (b, h, i) in picks:
        hk = kv_head_of(h, Hq, Hkv)
        kb, vb = _widen(k[b, hk]), _widen(v[b, hk])
        qr = _widen(q[b, h, i:i + 1])
        br = None if bias is None else bias_of_row(bias, shape, b, h, i)
        sel = None if block_sel is None else sel_of_row(block_sel, shape, block_q, block_k, b, h, i)
        res.append(attention_rows(qr, kb, vb, np.array([i]), float(np.float64(scale)),
                                  causal_offset, window, key_valid_of(key_mask, b), softcap, br,
                                  None if sinks is None else float(np.float64(sinks[h])), sel)[0])
    return np.array(res)


def visible_pair_count(B, Hq, L, S, causal_offset, window, key_mask=None, row_block=1024,
                       block_sel=None, block_q=0, block_k=0) -> int:
    """Number of visible (query row, key) cells summed over all query heads, by building the
    explicit mask row block by row block."""
    total = 0
    if block_sel is not None:
        block_sel = np.broadcast_to(np.asarray(block_sel), (B, Hq, -(-L // block_q), -(-S // block_k)))
    for b in range(B):
        kv = None if key_mask is None else (key_mask[b] != 0)
        for r0 in range(0, L, row_block):
            rows = np.arange(r0, min(r0 + row_block, L))
            vis = visible(rows, S, causal_offset, window, kv)
            if block_sel is None:
                total += int(np.count_nonzero(vis)) * Hq
            else:
                for h in range(Hq):
                    total += int(np.count_nonzero(vis & block_selected(rows, S, block_sel[b, h], block_q, block_k)))
    return total


# ----------------------------------------------------------------------------------------------
# Brute force (pure Python scalars) for tiny cases
# ----------------------------------------------------------------------------------------------
def brute_sdpa(q, k, v, scale, causal_offset=NO_CAUSAL, window=0, key_mask=None, softcap=0.0, bias=None,
               sinks=None, block_sel=None, block_q=0, block_k=0):
    """Scalar-loop SDPA on nested lists / small arrays, with math.exp (and math.tanh for the
    soft-cap; bias: an array broadcastable to [B, Hq, L, S]; sinks: [Hq] logits; block_sel:
    indexed [b][h][i // block_q][j // block_k], broadcast over size-1 leading axes). Shapes as
    oracle_sdpa."""
    q, k, v = _widen(np.asarray(q)), _widen(np.asarray(k)), _widen(np.asarray(v))
    B, Hq, L, D = q.shape
    Hkv, S, Dv = k.shape[1], k.shape[2], v.shape[3]
    G = Hq // Hkv
    out = np.zeros((B, Hq, L, Dv))
    if bias is not None:
        bias = np.broadcast_to(np.asarray(bias, dtype=np.float64), (B, Hq, L, S))
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            for i in range(L):
                keys = []
                for j in range(S):
                    if causal_offset >= 0 and j > i + causal_offset:
                        continue
                    if causal_offset >= 0 and window > 0 and j < i + causal_offset - window + 1:
                        continue
                    if key_mask is not None and not key_mask[b][j]:
                        continue
                    if block_sel is not None:
                        sb = block_sel[b if len(block_sel) > 1 else 0]
                        sb = sb[h if len(sb) > 1 else 0]
                        if not sb[i // block_q][j // block_k]:
                            continue
                    s = 0.0
                    for d in range(D):
                        s += float(q[b, h, i, d]) * float(k[b, hk, j, d])
                    s = float(scale) * s
                    if softcap > 0.0:
                        s = softcap * math.tanh(s / softcap)
                    if bias is not None:
                        s = s + float(bias[b, h, i, j])
                        if s == -math.inf:
                            continue
                    keys.append((j, s))
                if not keys:
                    continue
                mx = max(s for _, s in keys)
                if sinks is not None:
                    mx = max(mx, float(sinks[h]))
                w = [(j, math.exp(s - mx)) for j, s in keys]
                tot = sum(x for _, x in w)
                if sinks is not None:
                    tot += math.exp(float(sinks[h]) - mx)
                for d in range(Dv):
                    out[b, h, i, d] = sum(x * float(v[b, hk, j, d]) for j, x in w) / tot
    return out


def host_workers() -> int:
    """Threads the oracle's timing mode uses: the cores in this process's affinity mask."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1
