"""Pins of the packed variable-length oracle (CPU only). Each pin ties ``oracle_varlen`` to
something other than itself: the dense oracle (pinned on its own in test_oracle.py), closed-form
visible-pair counts, scalar brute force on tiny inputs and structural invariants; planted mistakes
in the varlen oracle must turn at least one pin red."""
import numpy as np
import pytest

import oracle.sdpa as osdpa
import oracle.varlen as ovl
from oracle import NO_CAUSAL, brute_sdpa, oracle_sdpa, oracle_varlen
from workloads import make_varlen_inputs


def to_dense(x, s0, s1):
    """Rows [s0, s1) of a packed [total, H, D] array as a dense [1, H, n, D] array."""
    return np.ascontiguousarray(np.transpose(x[s0:s1], (1, 0, 2))[None])


def pin_single_sequence_is_dense():
    """One packed sequence is the dense call with causal_offset = Lk - Lq (and bidirectional /
    windowed likewise)."""
    for lq, lk, causal, window in [(33, 47, True, 0), (40, 40, True, 0), (17, 80, True, 9),
                                   (25, 60, False, 0), (64, 64, True, 1)]:
        x = make_varlen_inputs("varlen_chunks_b5", seed=3, lengths_q=[lq], lengths_k=[lk])
        got = oracle_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], x["scale"], causal, window)
        ref = oracle_sdpa(to_dense(x["q"], 0, lq), to_dense(x["k"], 0, lk), to_dense(x["v"], 0, lk), x["scale"],
                          causal_offset=(lk - lq) if causal else NO_CAUSAL, window=window)
        assert np.allclose(np.transpose(got, (1, 0, 2)), ref[0], atol=1e-12, rtol=0)


def pin_equal_length_pair_count():
    """Lq == Lk: local row i sees local keys 0..i (the page's rule (k - cu_k) <= (q - cu_q)), so a
    sequence has Lq (Lq + 1) / 2 visible cells; with a window W, sum_i min(i + 1, W)."""
    for L in (1, 2, 7, 64, 65, 130):
        assert int(ovl.varlen_visible(L, L, True, 0).sum()) == L * (L + 1) // 2
        for W in (1, 5, 64):
            assert int(ovl.varlen_visible(L, L, True, W).sum()) == sum(min(i + 1, W) for i in range(L))
    assert int(ovl.varlen_visible(5, 9, False, 0).sum()) == 45


def pin_more_rows_than_keys():
    """Lq > Lk: the rows are the last Lq positions, so local row i sees keys 0..i - (Lq - Lk): the
    first Lq - Lk rows see nothing (zeros) and every other row equals bidirectional attention over
    the truncated key prefix (scalar brute force)."""
    lq, lk = 6, 3
    x = make_varlen_inputs("varlen_chunks_b5", seed=5, lengths_q=[lq], lengths_k=[lk], D=4, Hq=2, Hkv=1)
    got = oracle_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], x["scale"], True, 0)
    assert np.all(got[: lq - lk] == 0.0)
    for i in range(lq - lk, lq):
        n = i - (lq - lk) + 1
        ref = brute_sdpa(to_dense(x["q"], i, i + 1), to_dense(x["k"], 0, n), to_dense(x["v"], 0, n), x["scale"])
        assert np.allclose(got[i], ref[0, :, 0], atol=1e-12, rtol=0)


def pin_brute_force_ragged():
    """Three tiny ragged sequences (one with more keys than rows, one equal, one empty of rows)
    against scalar brute force per sequence, GQA 4:2."""
    lq, lk = [3, 4, 0], [5, 4, 2]
    x = make_varlen_inputs("varlen_chunks_b5", seed=11, lengths_q=lq, lengths_k=lk, D=4, Hq=4, Hkv=2)
    got = oracle_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], x["scale"], True, 0)
    cq, ck = x["cu_q"], x["cu_k"]
    for b in range(3):
        if lq[b] == 0:
            continue
        ref = brute_sdpa(to_dense(x["q"], cq[b], cq[b + 1]), to_dense(x["k"], ck[b], ck[b + 1]),
                         to_dense(x["v"], ck[b], ck[b + 1]), x["scale"], causal_offset=lk[b] - lq[b])
        assert np.allclose(np.transpose(got[cq[b]:cq[b + 1]], (1, 0, 2)), ref[0], atol=1e-12, rtol=0)


def pin_sequences_independent():
    """No attention across sequences: changing another sequence's data leaves a sequence's output
    unchanged, and a sequence with no keys outputs zeros."""
    lq, lk = [5, 7, 4], [9, 7, 0]
    x = make_varlen_inputs("varlen_chunks_b5", seed=13, lengths_q=lq, lengths_k=lk, D=8, Hq=2, Hkv=2)
    base = oracle_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], x["scale"], True, 0)
    cq, ck = x["cu_q"], x["cu_k"]
    k2, v2 = x["k"].copy(), x["v"].copy()
    k2[ck[1]:ck[2]] ^= np.uint16(0x0040)  # perturb sequence 1's keys and values only
    v2[ck[1]:ck[2]] ^= np.uint16(0x0040)
    got = oracle_varlen(x["q"], k2, v2, cq, ck, x["scale"], True, 0)
    assert np.array_equal(got[cq[0]:cq[1]], base[cq[0]:cq[1]])
    assert not np.allclose(got[cq[1]:cq[2]], base[cq[1]:cq[2]])
    assert np.all(base[cq[2]:cq[3]] == 0.0)


def pin_options_match_dense():
    """With a soft-cap and sink logits, each packed sequence is the dense oracle on that sequence
    with the same options (pinned in test_oracle.py), and scalar brute force on tiny sequences."""
    lq, lk = [20, 33, 4], [50, 33, 9]  # Lk >= Lq: the dense offset Lk - Lq is a causal one
    x = make_varlen_inputs("varlen_chunks_b5", seed=17, lengths_q=lq, lengths_k=lk, D=16, Hq=4, Hkv=2)
    sinks = np.array([0.3, -1.0, 2.0, -np.inf])
    got = oracle_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], x["scale"], True, 0, softcap=2.5, sinks=sinks)
    cq, ck = x["cu_q"], x["cu_k"]
    for b in range(3):
        ref = oracle_sdpa(to_dense(x["q"], cq[b], cq[b + 1]), to_dense(x["k"], ck[b], ck[b + 1]),
                          to_dense(x["v"], ck[b], ck[b + 1]), x["scale"], causal_offset=lk[b] - lq[b],
                          softcap=2.5, sinks=sinks)
        assert np.allclose(np.transpose(got[cq[b]:cq[b + 1]], (1, 0, 2)), ref[0], atol=1e-12, rtol=0)
    y = make_varlen_inputs("varlen_chunks_b5", seed=19, lengths_q=[3, 2], lengths_k=[4, 2], D=4, Hq=2, Hkv=1)
    got = oracle_varlen(y["q"], y["k"], y["v"], y["cu_q"], y["cu_k"], y["scale"], True, 0, softcap=1.5,
                        sinks=sinks[:2])
    for b, (a0, a1, k0, k1) in enumerate([(0, 3, 0, 4), (3, 5, 4, 6)]):
        ref = brute_sdpa(to_dense(y["q"], a0, a1), to_dense(y["k"], k0, k1), to_dense(y["v"], k0, k1), y["scale"],
                         causal_offset=(k1 - k0) - (a1 - a0), softcap=1.5, sinks=sinks[:2])
        assert np.allclose(np.transpose(got[a0:a1], (1, 0, 2)), ref[0], atol=1e-12, rtol=0)


def pin_selected_rows_match_full_oracle():
    """oracle_varlen_rows (one row at a time, used at full workload sizes) equals the matching rows
    of oracle_varlen for every (packed row, head) pair, on batches with sequences without rows,
    sequences without keys, more rows than keys, a last sequence, windows, soft-cap and sinks."""
    rng = np.random.default_rng(99)
    Hq, Hkv, D = 4, 2, 8
    for lq, lk, causal, window, softcap, sinks in [
            ([5, 0, 4, 3], [7, 3, 4, 0], True, 0, 0.0, None),
            ([3, 6, 0, 2], [3, 2, 5, 9], True, 3, 2.5, rng.standard_normal(Hq)),
            ([0, 4, 4, 1], [2, 4, 0, 6], False, 0, 0.0, rng.standard_normal(Hq))]:
        cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
        cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
        q = rng.standard_normal((int(cu_q[-1]), Hq, D))
        k = rng.standard_normal((int(cu_k[-1]), Hkv, D))
        v = rng.standard_normal((int(cu_k[-1]), Hkv, D))
        full = oracle_varlen(q, k, v, cu_q, cu_k, 0.6, causal, window, softcap, sinks)
        picks = [(r, h) for r in range(int(cu_q[-1])) for h in range(Hq)]
        rows = ovl.oracle_varlen_rows(q, k, v, cu_q, cu_k, 0.6, causal, window, picks, softcap, sinks)
        want = np.array([full[r, h] for (r, h) in picks])
        assert np.allclose(rows, want, atol=1e-12, rtol=0), (lq, lk)
        assert np.count_nonzero(np.abs(want).sum(axis=1)) > len(picks) // 3  # not vacuous


PINS = [pin_single_sequence_is_dense, pin_equal_length_pair_count, pin_more_rows_than_keys,
        pin_brute_force_ragged, pin_sequences_independent, pin_options_match_dense,
        pin_selected_rows_match_full_oracle]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_varlen_pin(pin):
    pin()


def test_varlen_generator_is_seeded_and_packed():
    a = make_varlen_inputs("varlen_chunks_b5", seed=0)
    b = make_varlen_inputs("varlen_chunks_b5", seed=0)
    assert all(np.array_equal(a[k], b[k]) for k in ("q", "k", "v", "cu_q", "cu_k"))
    assert a["cu_q"][0] == 0 and a["cu_q"][-1] == a["total_q"] == a["q"].shape[0]
    assert a["cu_k"][-1] == a["total_k"] == a["k"].shape[0]
    assert np.all(np.diff(a["cu_q"]) >= 1) and np.all(np.diff(a["cu_k"]) >= np.diff(a["cu_q"]))
    assert a["q"].shape[1:] == (8, 128) and a["k"].shape[1:] == (2, 128)
    c = make_varlen_inputs("varlen_causal_b8", seed=0)
    assert np.array_equal(c["cu_q"], c["cu_k"]) and 1024 <= c["lengths_q"].min() <= c["lengths_q"].max() <= 4096


# ---- planted mistakes (in the oracle, on the CPU) ----
_vis_orig = ovl.varlen_visible


def _bad_upper_left(Lq, Lk, causal, window):
    # ignore the per-sequence offset (upper-left causal)
    i = np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    v = np.ones((Lq, Lk), dtype=bool)
    if causal:
        v &= j <= i
        if window > 0:
            v &= j >= i - window + 1
    return v


def _bad_causal_plus_one(Lq, Lk, causal, window):
    v = _vis_orig(Lq, Lk, causal, window)
    if causal and Lk > 0 and Lq > 0:
        v = v | np.eye(Lq, Lk, k=Lk - Lq + 1, dtype=bool)
    return v


def _bad_window(Lq, Lk, causal, window):
    return _vis_orig(Lq, Lk, causal, window + 1 if window > 0 else window)


def _bad_head_map(h, Hq, Hkv):
    return h % Hkv


def _bad_sequence_left(cu_q, r):
    # the leftmost prefix sum <= r: a row right after a sequence without rows goes to that sequence
    return int(np.searchsorted(np.asarray(cu_q, dtype=np.int64), r, side="left") - 1) if r > 0 else 0


def _bad_sequence_off_by_one(cu_q, r):
    return max(0, _seq_orig(cu_q, r) - 1)


_seq_orig = ovl.sequence_of_row


@pytest.mark.parametrize("mod,attr,bad", [(ovl, "varlen_visible", _bad_upper_left),
                                          (ovl, "varlen_visible", _bad_causal_plus_one),
                                          (ovl, "varlen_visible", _bad_window),
                                          (ovl, "kv_head_of", _bad_head_map),
                                          (ovl, "sequence_of_row", _bad_sequence_left),
                                          (ovl, "sequence_of_row", _bad_sequence_off_by_one)],
                         ids=["upper_left", "causal_plus_one", "window_plus_one", "head_map_mod",
                              "rows_sequence_side_left", "rows_sequence_off_by_one"])
def test_varlen_planted_mistake_is_caught(monkeypatch, mod, attr, bad):
    monkeypatch.setattr(mod, attr, bad)
    caught = 0
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                caught += 1
    assert caught >= 1, f"no pin caught the planted mistake in {attr}"
