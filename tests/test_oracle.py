"""Pins for the CPU oracle: page-printed values, closed forms, invariants, brute force and a
library cross-check, plus planted mistakes that each pin must catch. CPU only."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.sdpa as osdpa
from oracle import brute_sdpa, oracle_sdpa, visible, visible_pair_count
from workloads import CONFIGS, f32_to_bf16_bits, make_inputs

RNG = np.random.default_rng(1234)


def rand(shape, rng=None):
    rng = RNG if rng is None else rng
    return rng.standard_normal(shape)


# ----------------------------------------------------------------------------------------------
# Pins written as plain functions so that the planted-mistake tests can re-run them.
# ----------------------------------------------------------------------------------------------
def pin_two_key_sigmoid():
    """Textbook: with two visible keys, softmax weights are (1 - s, s) with s = sigmoid(d1 - d0),
    so o = v0 + sigmoid(scale*(q.k1 - q.k0)) (v1 - v0)."""
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    q = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    k = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    v = np.array([[[[1.0, 2.0], [3.0, 4.0]]]])
    v0, v1 = v[0, 0, 0], v[0, 0, 1]
    # causal, offset 0: row 0 sees key 0 only, row 1 sees both keys
    o = oracle_sdpa(q, k, v, 1.0, causal_offset=0)
    assert np.allclose(o[0, 0, 0], v0, atol=1e-14, rtol=0)
    assert np.allclose(o[0, 0, 1], v0 + sig(1.0) * (v1 - v0), atol=1e-14, rtol=0)
    assert np.allclose(o[0, 0, 1], [2.4621171572600098, 3.4621171572600098], atol=1e-12)
    # bidirectional: row 0 weights keys by (1, 0) scores
    o = oracle_sdpa(q, k, v, 1.0, causal_offset=-1)
    assert np.allclose(o[0, 0, 0], v0 + sig(-1.0) * (v1 - v0), atol=1e-14, rtol=0)
    assert np.allclose(o[0, 0, 0], [1.5378828427399902, 2.5378828427399902], atol=1e-12)
    assert np.allclose(o[0, 0, 1], v0 + sig(1.0) * (v1 - v0), atol=1e-14, rtol=0)
    # a non-unit scale and general vectors
    rng = np.random.default_rng(7)
    for _ in range(5):
        D = 3
        q = rng.standard_normal((1, 1, 1, D))
        k = rng.standard_normal((1, 1, 2, D))
        v = rng.standard_normal((1, 1, 2, D))
        scale = 0.37
        d = scale * (q[0, 0, 0] @ k[0, 0, 1] - q[0, 0, 0] @ k[0, 0, 0])
        ref = v[0, 0, 0] + sig(d) * (v[0, 0, 1] - v[0, 0, 0])
        o = oracle_sdpa(q, k, v, scale, causal_offset=-1)
        assert np.allclose(o[0, 0, 0], ref, atol=1e-13, rtol=0)


def pin_rows_sum_to_one():
    """V = identity turns the output into the probability matrix: every non-empty row sums to 1
    and masked keys get exactly zero weight."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, L, S = 2, 4, 2, 7, 11
    q = rng.standard_normal((B, Hq, L, 8))
    k = rng.standard_normal((B, Hkv, S, 8))
    eye = np.broadcast_to(np.eye(S), (B, Hkv, S, S)).copy()
    km = (rng.random((B, S)) < 0.7).astype(np.uint8)
    for off, W in [(4, 0), (6, 3), (-1, 0), (0, 0), (20, 0)]:
        P = oracle_sdpa(q, k, eye, 0.5, off, W, km)
        for b in range(B):
            vis = visible(np.arange(L), S, off, W, km[b] != 0)
            for h in range(Hq):
                assert np.all(P[b, h][~vis] == 0.0)
                nonempty = vis.any(axis=1)
                assert np.allclose(P[b, h][nonempty].sum(axis=1), 1.0, atol=1e-12)
                assert np.all(P[b, h][~nonempty] == 0.0)


def pin_uniform_v_returns_v():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, L, S, D = 1, 6, 3, 9, 30, 5
    q = rng.standard_normal((B, Hq, L, D)) * 3
    k = rng.standard_normal((B, Hkv, S, D)) * 3
    c = rng.standard_normal((B, Hkv, 1, D))
    v = np.broadcast_to(c, (B, Hkv, S, D)).copy()
    o = oracle_sdpa(q, k, v, 0.9, 21, 5, None)
    for h in range(Hq):
        assert np.allclose(o[0, h], c[0, h // 2, 0][None, :], atol=1e-13)


def pin_window_reductions():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, L, S, D = 1, 2, 1, 6, 13, 4
    q, k, v = rng.standard_normal((B, Hq, L, D)), rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    off = S - L
    causal = oracle_sdpa(q, k, v, 0.5, off, 0)
    for W in (S + off, S + off + 5, 10 ** 6):
        assert np.array_equal(oracle_sdpa(q, k, v, 0.5, off, W), causal)
    # a window of one key: each row sees exactly its own position
    o1 = oracle_sdpa(q, k, v, 0.5, off, 1)
    for i in range(L):
        assert np.allclose(o1[0, :, i], v[0, 0, i + off][None, :], atol=1e-15, rtol=0)
    # window of two keys: a two-key softmax over positions i+off-1 and i+off
    o2 = oracle_sdpa(q, k, v, 0.5, off, 2)
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    for i in range(L):
        j0, j1 = i + off - 1, i + off
        d = 0.5 * (q[0, 0, i] @ k[0, 0, j1] - q[0, 0, i] @ k[0, 0, j0])
        assert np.allclose(o2[0, 0, i], v[0, 0, j0] + sig(d) * (v[0, 0, j1] - v[0, 0, j0]), atol=1e-13)


def pin_gqa_is_expanded_mha():
    rng = np.random.default_rng(6)
    for G in (2, 3, 7):
        B, Hkv, L, S, D = 2, 2, 5, 9, 4
        Hq = G * Hkv
        q = rng.standard_normal((B, Hq, L, D))
        k = rng.standard_normal((B, Hkv, S, D))
        v = rng.standard_normal((B, Hkv, S, D))
        o = oracle_sdpa(q, k, v, 0.7, 4, 0)
        o_mha = oracle_sdpa(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.7, 4, 0)
        assert np.array_equal(o, o_mha)
        # each head equals a single-head call on its own KV head h // G
        for h in range(Hq):
            oh = oracle_sdpa(q[:, h:h + 1], k[:, h // G:h // G + 1], v[:, h // G:h // G + 1], 0.7, 4, 0)
            assert np.array_equal(o[:, h:h + 1], oh)


def pin_triu_counts():
    """tinygrad's prefill mask full((T, sp+T), -inf).triu(sp+1) for T in 2..5, sp in {0,2,5}:
    visible (finite) = T*sp + T(T+1)/2, masked = T(T-1)/2, total = T*(sp+T)."""
    for T in range(2, 6):
        for sp in (0, 2, 5):
            vis = visible(np.arange(T), sp + T, sp, 0, None)
            assert vis.size == T * (sp + T)
            assert int(vis.sum()) == T * sp + T * (T + 1) // 2
            assert int((~vis).sum()) == T * (T - 1) // 2
            # the masked cells are exactly the strict upper triangle shifted by sp (triu(sp+1))
            tri = np.triu(np.ones((T, sp + T), dtype=bool), sp + 1)
            assert np.array_equal(~vis, tri)


def pin_zero_scale_prefix_means():
    """scale = 0 makes all visible keys equally likely: row i is the mean of V over its visible
    range, which a cumulative sum gives directly."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, L, S, D = 1, 2, 1, 8, 20, 3
    q, k, v = rng.standard_normal((B, Hq, L, D)), rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    csum = np.concatenate([np.zeros((1, D)), np.cumsum(v[0, 0], axis=0)])
    for off, W in [(12, 0), (12, 4), (3, 0), (0, 2)]:
        o = oracle_sdpa(q, k, v, 0.0, off, W)
        for i in range(L):
            hi = min(S - 1, i + off)
            lo = max(0, i + off - W + 1) if W > 0 else 0
            ref = (csum[hi + 1] - csum[lo]) / (hi - lo + 1)
            assert np.allclose(o[0, 0, i], ref, atol=1e-13), (off, W, i)
    n = 13
    km = (np.arange(S) < n).astype(np.uint8)[None, :]
    o = oracle_sdpa(q, k, v, 0.0, -1, 0, km)
    assert np.allclose(o[0, 1], (csum[n] / n)[None, :], atol=1e-13)


def pin_chunk_equals_tail():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, S, D = 1, 4, 2, 17, 6
    q_full = rng.standard_normal((B, Hq, S, D))
    k, v = rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    full = oracle_sdpa(q_full, k, v, 0.4, 0, 0)
    for L in (1, 5, 17):
        chunk = oracle_sdpa(q_full[:, :, S - L:], k, v, 0.4, S - L, 0)
        assert np.allclose(chunk, full[:, :, S - L:], atol=1e-14, rtol=0)


def pin_key_padding():
    rng = np.random.default_rng(10)
    B, Hq, Hkv, L, S, D = 2, 2, 1, 6, 15, 4
    q, k, v = rng.standard_normal((B, Hq, L, D)), rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    lens = [9, 15]
    km = (np.arange(S)[None, :] < np.array(lens)[:, None]).astype(np.uint8)
    o = oracle_sdpa(q, k, v, 0.3, -1, 0, km)
    for b, n in enumerate(lens):
        ot = oracle_sdpa(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.3, -1, 0)
        assert np.allclose(o[b:b + 1], ot, atol=1e-14, rtol=0)
    ones = np.ones((B, S), dtype=np.uint8)
    assert np.array_equal(oracle_sdpa(q, k, v, 0.3, 7, 0, ones), oracle_sdpa(q, k, v, 0.3, 7, 0))
    # all keys masked (tiny-llm Task 2's 9 x 17 witness): finite, all-zero output
    q9, k17, v17 = rng.standard_normal((1, 2, 9, 4)), rng.standard_normal((1, 1, 17, 4)), rng.standard_normal((1, 1, 17, 4))
    o = oracle_sdpa(q9, k17, v17, 0.5, -1, 0, np.zeros((1, 17), dtype=np.uint8))
    assert np.all(o == 0.0) and np.all(np.isfinite(o))


def pin_brute_force():
    """The vectorised oracle equals an independent scalar-loop implementation on small cases."""
    rng = np.random.default_rng(11)
    cases = [(1, 4, 2, 5, 9, 4, 4, 0, False), (2, 3, 1, 4, 4, 3, 0, 0, True),
             (1, 2, 2, 6, 13, 2, 7, 3, True), (1, 2, 1, 3, 8, 5, -1, 0, True),
             (1, 6, 2, 7, 7, 3, 0, 1, False), (1, 2, 1, 9, 5, 2, 0, 0, False)]
    for B, Hq, Hkv, L, S, D, off, W, use_mask in cases:
        q = rng.standard_normal((B, Hq, L, D))
        k = rng.standard_normal((B, Hkv, S, D))
        v = rng.standard_normal((B, Hkv, S, D))
        km = (rng.random((B, S)) < 0.6).astype(np.uint8) if use_mask else None
        o = oracle_sdpa(q, k, v, 0.6, off, W, km, row_block=2)
        ob = brute_sdpa(q, k, v, 0.6, off, W, km)
        assert np.allclose(o, ob, atol=1e-13, rtol=0), (B, Hq, Hkv, L, S, D, off, W)



def pin_softcap():
    """Logit soft-capping (brotensor attn_softcap): the two-key sigmoid identity on capped scores,
    scalar brute force (math.tanh) on random masked cases, the large-cap limit (no cap) and the
    small-cap limit (capped scores all near 0: the mean of the visible values)."""
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    rng = np.random.default_rng(17)
    for cap in (0.5, 2.0, 30.0):
        q = rng.standard_normal((1, 1, 1, 3))
        k = rng.standard_normal((1, 1, 2, 3)) * 4.0
        v = rng.standard_normal((1, 1, 2, 3))
        scale = 0.8
        s0, s1 = scale * float(q[0, 0, 0] @ k[0, 0, 0]), scale * float(q[0, 0, 0] @ k[0, 0, 1])
        d = cap * math.tanh(s1 / cap) - cap * math.tanh(s0 / cap)
        ref = v[0, 0, 0] + sig(d) * (v[0, 0, 1] - v[0, 0, 0])
        got = oracle_sdpa(q, k, v, scale, causal_offset=-1, softcap=cap)
        assert np.allclose(got[0, 0, 0], ref, atol=1e-13, rtol=0)
    for cap, off, W in [(1.0, 2, 0), (5.0, 0, 3), (0.3, -1, 0)]:
        q = rng.standard_normal((1, 2, 4, 5)) * 3.0
        k = rng.standard_normal((1, 1, 6, 5))
        v = rng.standard_normal((1, 1, 6, 5))
        got = oracle_sdpa(q, k, v, 0.6, causal_offset=off, window=W, softcap=cap)
        ref = brute_sdpa(q, k, v, 0.6, causal_offset=off, window=W, softcap=cap)
        assert np.allclose(got, ref, atol=1e-12, rtol=0)
    q = rng.standard_normal((1, 2, 8, 16))
    k = rng.standard_normal((1, 2, 20, 16))
    v = rng.standard_normal((1, 2, 20, 16))
    plain = oracle_sdpa(q, k, v, 0.25, causal_offset=12)
    assert np.allclose(oracle_sdpa(q, k, v, 0.25, causal_offset=12, softcap=1e7), plain, atol=1e-10, rtol=0)
    tiny = oracle_sdpa(q, k, v, 0.25, causal_offset=12, softcap=1e-9)
    for i in range(8):
        assert np.allclose(tiny[0, :, i], v[0, :, : i + 13].mean(axis=1), atol=1e-7, rtol=0)


def pin_additive_bias():
    """Additive bias (tiny-llm Task 2): zero bias is no bias; a -inf bias equals the key mask; a
    per-row constant cancels (softmax shift invariance); the two-key sigmoid identity on biased
    scores; scalar brute force with broadcast biases and the causal term."""
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    rng = np.random.default_rng(23)
    q = rng.standard_normal((2, 2, 6, 8))
    k = rng.standard_normal((2, 1, 10, 8))
    v = rng.standard_normal((2, 1, 10, 8))
    plain = oracle_sdpa(q, k, v, 0.4, causal_offset=4)
    assert np.array_equal(oracle_sdpa(q, k, v, 0.4, causal_offset=4, bias=np.zeros((6, 10))), plain)
    km = (rng.random((2, 10)) > 0.4).astype(np.uint8)
    km[:, 0] = 1
    neg = np.where(km[:, None, None, :] != 0, 0.0, -np.inf)
    assert np.allclose(oracle_sdpa(q, k, v, 0.4, causal_offset=4, bias=neg),
                       oracle_sdpa(q, k, v, 0.4, causal_offset=4, key_mask=km), atol=1e-14, rtol=0)
    rowc = rng.standard_normal((2, 2, 6, 1)) * 5.0
    assert np.allclose(oracle_sdpa(q, k, v, 0.4, causal_offset=4, bias=np.broadcast_to(rowc, (2, 2, 6, 10))),
                       plain, atol=1e-12, rtol=0)
    q1 = rng.standard_normal((1, 1, 1, 3))
    k1 = rng.standard_normal((1, 1, 2, 3))
    v1 = rng.standard_normal((1, 1, 2, 3))
    bb = np.array([[[[0.7, -1.9]]]])
    d = 0.5 * float(q1[0, 0, 0] @ k1[0, 0, 1]) - 1.9 - 0.5 * float(q1[0, 0, 0] @ k1[0, 0, 0]) - 0.7
    ref = v1[0, 0, 0] + sig(d) * (v1[0, 0, 1] - v1[0, 0, 0])
    assert np.allclose(oracle_sdpa(q1, k1, v1, 0.5, causal_offset=-1, bias=bb)[0, 0, 0], ref, atol=1e-13, rtol=0)
    for shape in [(6, 10), (2, 1, 6, 10), (1, 2, 1, 10)]:
        bias = rng.standard_normal(shape) * 2.0
        got = oracle_sdpa(q, k, v, 0.4, causal_offset=4, window=3, bias=bias, softcap=1.5)
        ref = brute_sdpa(q, k, v, 0.4, causal_offset=4, window=3, bias=bias, softcap=1.5)
        assert np.allclose(got, ref, atol=1e-12, rtol=0)


def pin_sinks():
    """Attention sinks (one logit per query head, an extra softmax term with no value): a -inf
    sink is no sink; with all scores 0 and uniform values c, a row with n visible keys gives
    c n / (n + e^sink) (per query head, not per KV head); one visible key of score s gives
    V sigmoid(s - sink) (the sink is not scaled); a row without visible keys stays 0; adding a
    constant to every score and to the sinks changes nothing; scalar brute force."""
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    rng = np.random.default_rng(29)
    q = rng.standard_normal((2, 4, 6, 8))
    k = rng.standard_normal((2, 2, 10, 8))
    v = rng.standard_normal((2, 2, 10, 8))
    plain = oracle_sdpa(q, k, v, 0.4, causal_offset=4)
    assert np.array_equal(oracle_sdpa(q, k, v, 0.4, causal_offset=4, sinks=np.full(4, -np.inf)), plain)
    sinks = np.array([-1.0, 0.5, 2.0, math.log(3.0)])
    c = rng.standard_normal((2, 2, 1, 8))
    o = oracle_sdpa(q, np.zeros_like(k), np.broadcast_to(c, v.shape), 0.4, causal_offset=4, sinks=sinks)
    for h in range(4):
        for i in range(6):
            n = i + 4 + 1
            assert np.allclose(o[:, h, i], c[:, h // 2, 0] * n / (n + math.exp(sinks[h])), atol=1e-14, rtol=0)
    q1 = rng.standard_normal((1, 1, 1, 3))
    k1 = rng.standard_normal((1, 1, 1, 3))
    v1 = rng.standard_normal((1, 1, 1, 3))
    s1 = 0.5 * float(q1[0, 0, 0] @ k1[0, 0, 0])
    got = oracle_sdpa(q1, k1, v1, 0.5, causal_offset=0, sinks=np.array([1.25]))[0, 0, 0]
    assert np.allclose(got, v1[0, 0, 0] * sig(s1 - 1.25), atol=1e-14, rtol=0)
    km = np.ones((2, 10), dtype=np.uint8)
    km[1, :] = 0
    o = oracle_sdpa(q, k, v, 0.4, key_mask=km, sinks=sinks)
    assert np.all(o[1] == 0.0) and np.all(np.isfinite(o))
    shifted = oracle_sdpa(q, k, v, 0.4, causal_offset=4, sinks=sinks + 3.5, bias=np.full((6, 10), 3.5))
    assert np.allclose(shifted, oracle_sdpa(q, k, v, 0.4, causal_offset=4, sinks=sinks), atol=1e-13, rtol=0)
    bias = rng.standard_normal((1, 4, 6, 10))
    got = oracle_sdpa(q, k, v, 0.4, causal_offset=4, window=3, softcap=1.5, bias=bias, sinks=sinks)
    ref = brute_sdpa(q, k, v, 0.4, causal_offset=4, window=3, softcap=1.5, bias=bias, sinks=sinks)
    assert np.allclose(got, ref, atol=1e-12, rtol=0)


def pin_block_bitmap():
    """Block bitmap: an all-ones bitmap is no bitmap; a block-diagonal bitmap without the causal
    term is independent attention inside each block; the bitmap equals the -inf additive bias of
    its element-wise expansion (built with a Kronecker product); K = 0 with a ramp in V gives the
    mean visible key index, worked by hand; scalar brute force with per-head bitmaps, the causal
    term and a window."""
    rng = np.random.default_rng(31)
    q = rng.standard_normal((2, 4, 12, 8))
    k = rng.standard_normal((2, 2, 12, 8))
    v = rng.standard_normal((2, 2, 12, 8))
    plain = oracle_sdpa(q, k, v, 0.4, causal_offset=0)
    ones = np.ones((1, 1, 3, 3), dtype=np.uint8)
    assert np.array_equal(oracle_sdpa(q, k, v, 0.4, causal_offset=0, block_sel=ones, block_q=4, block_k=4), plain)
    diag = np.eye(3, dtype=np.uint8)[None, None]
    o = oracle_sdpa(q, k, v, 0.4, block_sel=diag, block_q=4, block_k=4)
    for r in range(3):
        sl = slice(4 * r, 4 * r + 4)
        assert np.allclose(o[:, :, sl], oracle_sdpa(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.4), atol=1e-13, rtol=0)
    L, S, bq, bk = 12, 12, 4, 6
    sel = (rng.random((2, 4, 3, 2)) > 0.4).astype(np.uint8)
    dense = np.kron(sel, np.ones((bq, bk), dtype=np.uint8))[..., :L, :S]
    neg = np.where(dense != 0, 0.0, -np.inf)
    got = oracle_sdpa(q, k, v, 0.4, causal_offset=0, block_sel=sel, block_q=bq, block_k=bk)
    ref = oracle_sdpa(q, k, v, 0.4, causal_offset=0, bias=neg)
    assert np.allclose(got, ref, atol=1e-14, rtol=0)
    # L = 4 rows, S = 8 keys, blocks of 2 rows x 4 keys, bitmap [[1, 0], [0, 1]], no causal term:
    # rows 0-1 see keys 0-3 (mean index 1.5), rows 2-3 see keys 4-7 (mean index 5.5)
    vr = np.zeros((1, 1, 8, 2))
    vr[0, 0, :, 0] = np.arange(8)
    o = oracle_sdpa(rng.standard_normal((1, 1, 4, 2)), np.zeros((1, 1, 8, 2)), vr, 1.0,
                    block_sel=np.array([[[[1, 0], [0, 1]]]]), block_q=2, block_k=4)
    assert np.allclose(o[0, 0, :, 0], [1.5, 1.5, 5.5, 5.5], atol=1e-14, rtol=0)
    kk = rng.standard_normal((2, 2, 11, 8))
    vv = rng.standard_normal((2, 2, 11, 8))
    sel = (rng.random((2, 4, 2, 4)) > 0.5).astype(np.uint8)
    got = oracle_sdpa(q[:, :, :7], kk, vv, 0.4, causal_offset=4, window=5, block_sel=sel, block_q=4, block_k=3)
    ref = brute_sdpa(q[:, :, :7], kk, vv, 0.4, causal_offset=4, window=5, block_sel=sel, block_q=4, block_k=3)
    assert np.allclose(got, ref, atol=1e-12, rtol=0)

def pin_selected_rows_match_full_oracle():
    """oracle_selected_rows (one row at a time, used at full workload sizes) equals the matching
    rows of oracle_sdpa on small cases with every option: per-batch key masks, causal offset and
    window, soft-cap, an additive bias broadcast as [L, S], [B, 1, L, S] and [1, Hq, 1, S], sinks
    and a per-(b, h) block bitmap with B > 1. Every (b, h, i) triple is picked."""
    rng = np.random.default_rng(2024)
    B, Hq, Hkv, L, S, D = 2, 4, 2, 9, 13, 8
    q, k, v = rng.standard_normal((B, Hq, L, D)), rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    km = (rng.random((B, S)) < 0.7).astype(np.uint8)
    km[:, 0] = 1
    picks = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(L)]
    sinks = rng.standard_normal(Hq)
    cases = [
        dict(causal_offset=4, window=5, key_mask=km, softcap=3.0),
        dict(causal_offset=4, window=0, key_mask=None, bias=rng.standard_normal((L, S))),
        dict(causal_offset=-1, window=0, key_mask=km, bias=rng.standard_normal((B, 1, L, S))),
        dict(causal_offset=6, window=0, key_mask=None, bias=rng.standard_normal((1, Hq, 1, S)), sinks=sinks),
        dict(causal_offset=4, window=7, key_mask=None, softcap=2.0, sinks=sinks,
             block_sel=(rng.random((B, Hq, 3, 4)) < 0.6).astype(np.uint8), block_q=3, block_k=4),
        dict(causal_offset=-1, window=0, key_mask=None,
             block_sel=(rng.random((B, 1, 3, 4)) < 0.5).astype(np.uint8), block_q=3, block_k=4),
    ]
    for c in cases:
        full = oracle_sdpa(q, k, v, 0.4, **c)
        opts = {kk: vv for kk, vv in c.items() if kk not in ("causal_offset", "window", "key_mask")}
        rows = oracle.oracle_selected_rows(q, k, v, 0.4, c["causal_offset"], c["window"], c["key_mask"], picks,
                                           **opts)
        want = np.array([full[b, h, i] for (b, h, i) in picks])
        assert np.allclose(rows, want, atol=1e-12, rtol=0), sorted(c)
        assert np.count_nonzero(np.abs(want).sum(axis=1)) > len(picks) // 2  # not vacuous


PINS = [pin_selected_rows_match_full_oracle, pin_sinks, pin_block_bitmap, pin_softcap, pin_additive_bias, pin_two_key_sigmoid, pin_rows_sum_to_one, pin_uniform_v_returns_v, pin_window_reductions,
        pin_gqa_is_expanded_mha, pin_triu_counts, pin_zero_scale_prefix_means, pin_chunk_equals_tail,
        pin_key_padding, pin_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------------------------
# Values printed on the pages
# ----------------------------------------------------------------------------------------------
def test_worked_example_L3_S7(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "causal_rows_L3_S7.json")))
    L, S = g["L"], g["S"]
    assert g["causal_offset"] == S - L
    vis = visible(np.arange(L), S, S - L, 0, None)
    assert list(np.nonzero(vis[0])[0]) == g["first_row_visible"]
    assert [int(np.nonzero(r)[0].max()) for r in vis] == g["last_visible_per_row"]
    assert all(np.nonzero(r)[0].min() == 0 for r in vis)


def test_rotating_cache_key_count(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "rotating_cache_keys.json")))
    c = CONFIGS["sliding_w1024_d128"]
    assert g["window"] - 1 + g["L"] == g["S"] == c["S"] and c["window"] == g["window"]
    # with causal_offset = W - 1 every row sees exactly W keys: [i, i + W - 1]
    rows = np.array([0, 1, 1000, 2047])
    vis = visible(rows, c["S"], c["causal_offset"], c["window"], None)
    for r, row in zip(rows, vis):
        nz = np.nonzero(row)[0]
        assert nz.min() == r and nz.max() == r + g["window"] - 1 and nz.size == g["window"]


def test_witness_shapes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "witnesses.json")))
    c = CONFIGS["causal_witness_33x47"]
    assert (c["L"], c["S"]) == (g["causal_gqa_witness"]["L"], g["causal_gqa_witness"]["S"])
    w = g["all_masked_witness"]
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 2, w["L"], 8))
    k = rng.standard_normal((1, 1, w["S"], 8))
    o = oracle_sdpa(q, k, k, 0.3, -1, 0, np.zeros((1, w["S"]), dtype=np.uint8))
    assert np.all(o == w["expected_output"])


# ----------------------------------------------------------------------------------------------
# Library cross-check and closed-form pair counts
# ----------------------------------------------------------------------------------------------
def test_torch_sdpa_crosscheck():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(12)
    for B, Hq, Hkv, L, S, D, off, W, use_mask in [(2, 4, 2, 9, 21, 16, 12, 0, False),
                                                  (1, 6, 3, 16, 40, 8, 24, 10, True),
                                                  (2, 4, 4, 12, 12, 8, -1, 0, True)]:
        q = rng.standard_normal((B, Hq, L, D))
        k = rng.standard_normal((B, Hkv, S, D))
        v = rng.standard_normal((B, Hkv, S, D))
        km = (np.arange(S)[None, :] < rng.integers(S // 2, S + 1, size=B)[:, None]).astype(np.uint8) if use_mask else None
        o = oracle_sdpa(q, k, v, 0.25, off, W, km)
        G = Hq // Hkv
        masks = np.stack([visible(np.arange(L), S, off, W, None if km is None else km[b] != 0) for b in range(B)])
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(np.repeat(k, G, axis=1)),
            torch.from_numpy(np.repeat(v, G, axis=1)), attn_mask=torch.from_numpy(masks[:, None]),
            scale=0.25).numpy()
        nonempty = masks.any(axis=2)
        for b in range(B):
            assert np.allclose(o[b][:, nonempty[b]], ref[b][:, nonempty[b]], atol=1e-10, rtol=0)


def closed_form_pairs(L, S, off, W):
    """Visible pairs per head for causal(+window) masks, summed row by row in closed form."""
    total = 0
    for i in range(L):
        hi = min(S - 1, i + off) if off >= 0 else S - 1
        lo = max(0, i + off - W + 1) if (off >= 0 and W > 0) else 0
        total += max(0, hi - lo + 1)
    return total


@pytest.mark.parametrize("name,expected", [("causal_witness_33x47", 4092), ("small_prompt_128", 132096),
                                           ("mid_ctx_8k", 822140928), ("sliding_w1024_d128", 67108864),
                                           ("long_ctx_32k", 2080407552)])
def test_visible_pairs(name, expected):
    c = CONFIGS[name]
    per_head = closed_form_pairs(c["L"], c["S"], c["causal_offset"], c["window"])
    assert per_head * c["Hq"] * c["B"] == expected
    if c["L"] * c["S"] <= 4096 * 8192:
        assert visible_pair_count(c["B"], c["Hq"], c["L"], c["S"], c["causal_offset"], c["window"]) == expected


def test_padded_pairs_match_lengths():
    x = make_inputs("bidir_padded_b8", seed=0, Hq=1, L=8, D=4)
    n = x["key_lengths"]
    assert np.all((n >= 1024) & (n <= 4096))
    assert visible_pair_count(8, 1, 8, 4096, -1, 0, x["key_mask"]) == 8 * int(n.sum())


# ----------------------------------------------------------------------------------------------
# Input generator
# ----------------------------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # exact ties: low 16 bits = 0x8000, with both parities of the kept bit
    ties = (np.arange(1000, dtype=np.uint32) << np.uint32(17) | np.uint32(0x3F808000)).view(np.float32)
    ties2 = ((np.arange(1000, dtype=np.uint32) << np.uint32(17)) | np.uint32(0x3F818000)).view(np.float32)
    x = np.concatenate([x, ties, ties2, np.array([0.0, -0.0, 1e-40, -1e-40], dtype=np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # widening in the oracle is exact
    back = oracle.bf16_bits_to_f64(ours)
    assert np.array_equal(back, torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_generator_is_seeded_and_shaped():
    a = make_inputs("causal_witness_33x47", seed=0)
    b = make_inputs("causal_witness_33x47", seed=0)
    c = make_inputs("causal_witness_33x47", seed=1)
    for key in ("q", "k", "v"):
        assert np.array_equal(a[key], b[key]) and not np.array_equal(a[key], c[key])
    assert a["q"].shape == (1, 4, 33, 128) and a["k"].shape == (1, 2, 47, 128)
    assert a["scale"] == np.float32(1 / np.sqrt(np.float32(128)))
    s = make_inputs("small_prompt_128")
    qf = oracle.bf16_bits_to_f64(s["q"])
    assert 0.45 < qf.std() < 0.55  # N(0,1) * 0.5


# ----------------------------------------------------------------------------------------------
# Planted mistakes: each must turn at least one pin red (the mutation lives in the oracle, on CPU)
# ----------------------------------------------------------------------------------------------
def _bad_head_map(h, Hq, Hkv):
    return h % Hkv


def _bad_causal(rows, S, off, W, kv):
    return osdpa_visible_orig(rows, S, off + 1 if off >= 0 else off, W, kv)


def _bad_window(rows, S, off, W, kv):
    return osdpa_visible_orig(rows, S, off, W + 1 if W > 0 else W, kv)


def _bad_key_mask(rows, S, off, W, kv):
    return osdpa_visible_orig(rows, S, off, W, None)


osdpa_visible_orig = osdpa.visible


def _bad_scale(q_rows, k, v, rows, scale, off, W, kv, softcap=0.0, bias_rows=None, sink=None, sel_rows=None):
    return _attention_rows_orig(q_rows, k, v, rows, 1.0, off, W, kv, softcap, bias_rows, sink, sel_rows)


def _bad_softcap_after_mask(q_rows, k, v, rows, scale, off, W, kv, softcap=0.0, bias_rows=None, sink=None, sel_rows=None):
    # the soft-cap applied after the mask: masked keys (-inf) become -cap, i.e. visible
    S = k.shape[0]
    scores = float(scale) * (q_rows @ k.T) + osdpa.additive_mask(rows, S, off, W, kv)
    if bias_rows is not None:
        scores = scores + bias_rows
    if softcap > 0:
        scores = softcap * np.tanh(scores / softcap)
    if sel_rows is not None:
        scores = np.where(sel_rows, scores, -np.inf)
    return osdpa._softmax_rows_times_v(scores, v, sink)


def _bad_bias_ignored(q_rows, k, v, rows, scale, off, W, kv, softcap=0.0, bias_rows=None, sink=None, sel_rows=None):
    return _attention_rows_orig(q_rows, k, v, rows, scale, off, W, kv, softcap, None, sink, sel_rows)


def _bad_bias_sign(q_rows, k, v, rows, scale, off, W, kv, softcap=0.0, bias_rows=None, sink=None, sel_rows=None):
    return _attention_rows_orig(q_rows, k, v, rows, scale, off, W, kv, softcap,
                                None if bias_rows is None else -bias_rows, sink, sel_rows)


def _bad_softcap_unscaled(scores, softcap):
    # tanh of the score without dividing by the cap
    return softcap * np.tanh(scores) if softcap > 0 else scores


def _bad_sink_ignored(q_rows, k, v, rows, scale, off, W, kv, softcap=0.0, bias_rows=None, sink=None, sel_rows=None):
    return _attention_rows_orig(q_rows, k, v, rows, scale, off, W, kv, softcap, bias_rows, None, sel_rows)


def _bad_sink_scaled(q_rows, k, v, rows, scale, off, W, kv, softcap=0.0, bias_rows=None, sink=None, sel_rows=None):
    return _attention_rows_orig(q_rows, k, v, rows, scale, off, W, kv, softcap, bias_rows,
                                None if sink is None else sink * scale, sel_rows)


def _bad_sink_sign(q_rows, k, v, rows, scale, off, W, kv, softcap=0.0, bias_rows=None, sink=None, sel_rows=None):
    return _attention_rows_orig(q_rows, k, v, rows, scale, off, W, kv, softcap, bias_rows,
                                None if sink is None else -sink, sel_rows)


def _bad_sel_ignored(q_rows, k, v, rows, scale, off, W, kv, softcap=0.0, bias_rows=None, sink=None, sel_rows=None):
    return _attention_rows_orig(q_rows, k, v, rows, scale, off, W, kv, softcap, bias_rows, sink, None)


def _bad_sel_swapped_blocks(rows, S, sel_bh, block_q, block_k):
    # block sizes exchanged (indices clamped into the bitmap, so the mistake gives values, not errors)
    sel_bh = np.asarray(sel_bh)
    qb = np.minimum(np.asarray(rows, dtype=np.int64) // int(block_k), sel_bh.shape[0] - 1)
    kb = np.minimum(np.arange(S, dtype=np.int64) // int(block_q), sel_bh.shape[1] - 1)
    return sel_bh[qb][:, kb] != 0


def _bad_sel_transposed(rows, S, sel_bh, block_q, block_k):
    qb = np.asarray(rows, dtype=np.int64) // int(block_q)
    kb = np.arange(S, dtype=np.int64) // int(block_k)
    # bitmap read as [key block, query block] (indices clamped into it)
    t = np.asarray(sel_bh)
    return t[np.minimum(kb, t.shape[0] - 1)][:, np.minimum(qb, t.shape[1] - 1)].T != 0


_block_selected_orig = osdpa.block_selected


def _bad_empty_rows(scores, v, sink=None):
    m = np.max(scores, axis=1, keepdims=True)
    p = np.exp(scores - m)
    return (p @ v) / np.sum(p, axis=1, keepdims=True)


_attention_rows_orig = osdpa.attention_rows


def _bad_bias_first_row(bias, shape, b, h, i):
    # the bias row of query row 0 for every row
    return np.broadcast_to(np.asarray(bias, dtype=np.float64), shape)[b, h, 0:1]


def _bad_sel_batch0(block_sel, shape, block_q, block_k, b, h, i):
    # the bitmap of batch element 0 for every batch element
    B, Hq, L, S = shape
    full = np.broadcast_to(np.asarray(block_sel), (B, Hq, -(-L // block_q), -(-S // block_k)))
    return osdpa.block_selected(np.array([i]), S, full[0, h], block_q, block_k)


def _bad_key_valid_batch0(key_mask, b):
    return None if key_mask is None else (np.asarray(key_mask)[0] != 0)


@pytest.mark.parametrize("attr,bad", [("kv_head_of", _bad_head_map), ("visible", _bad_causal),
                                      ("visible", _bad_window), ("visible", _bad_key_mask),
                                      ("attention_rows", _bad_scale),
                                      ("_softmax_rows_times_v", _bad_empty_rows),
                                      ("attention_rows", _bad_softcap_after_mask),
                                      ("soft_cap", _bad_softcap_unscaled),
                                      ("attention_rows", _bad_bias_ignored),
                                      ("attention_rows", _bad_bias_sign),
                                      ("attention_rows", _bad_sink_ignored),
                                      ("attention_rows", _bad_sink_scaled),
                                      ("attention_rows", _bad_sink_sign),
                                      ("attention_rows", _bad_sel_ignored),
                                      ("block_selected", _bad_sel_swapped_blocks),
                                      ("block_selected", _bad_sel_transposed),
                                      ("bias_of_row", _bad_bias_first_row),
                                      ("sel_of_row", _bad_sel_batch0),
                                      ("key_valid_of", _bad_key_valid_batch0)],
                         ids=["head_map_mod", "causal_plus_one", "window_plus_one", "key_mask_dropped",
                              "scale_dropped", "empty_rows_nan", "softcap_after_mask", "softcap_unscaled",
                              "bias_ignored", "bias_sign", "sink_ignored", "sink_scaled", "sink_sign",
                              "sel_ignored", "sel_swapped_blocks", "sel_transposed",
                              "rows_bias_first_row", "rows_sel_batch0", "rows_key_mask_batch0"])
def test_planted_mistake_is_caught(monkeypatch, attr, bad):
    monkeypatch.setattr(osdpa, attr, bad)
    caught = 0
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                caught += 1
    assert caught >= 1, f"no pin caught the planted mistake in {attr}"


def test_generator_variant_draws():
    """Sinks and the block bitmap are drawn after Q, K, V: the value stream of Q, K, V is that of the
    plain workload; the bitmap keeps key block 0 and the block of each query block's last causal
    key, and selects about `density` of the rest."""
    plain = make_inputs("long_ctx_32k", seed=0, L=256, S=4096, causal_offset=3840, Hq=4, Hkv=1, D=8)
    for name in ("long_ctx_32k_sinks", "long_ctx_32k_sel"):
        x = make_inputs(name, seed=0, L=256, S=4096, causal_offset=3840, Hq=4, Hkv=1, D=8)
        for key in ("q", "k", "v"):
            assert np.array_equal(x[key], plain[key])
    s = make_inputs("long_ctx_32k_sinks", seed=0)
    assert s["sinks"].shape == (32,) and s["sinks"].dtype == np.float32
    x = make_inputs("long_ctx_32k_sel", seed=0)
    sel, bq, bk = x["block_sel"], x["block_q"], x["block_k"]
    assert sel.shape == (32, 16, 64) and (bq, bk) == (128, 512)
    assert np.all(sel[:, :, 0] == 1)
    for qb in range(16):
        assert np.all(sel[:, qb, (qb * 128 + 127 + 30720) // 512] == 1)
    assert 0.2 < sel.mean() < 0.35
