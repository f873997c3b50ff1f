"""Seeded sweep of random small shapes through the prefill and decode entry points against the fp64
CPU oracle: batch, group size, head dimension, query and key lengths (tails on both axes), causal
offset (bidirectional, zero, inside and beyond the keys), sliding window, key padding, soft-cap and
attention sinks drawn per case, so that combinations the enumerated tests do not list are covered.

Each case: |O_gpu - O_ref| <= 2e-2 + 2e-2 |O_ref| elementwise and rms(err)/rms(ref) <= 1e-2; rows
without a visible key are exact zeros; a prefill case is also run without tile skipping and must be
bit-identical.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import prefill_attention_amd as pfa  # noqa: E402
from oracle import NO_CAUSAL, oracle_sdpa  # noqa: E402
from workloads import make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

ATOL = RTOL = 2e-2
RMS_RATIO = 1e-2
DEV = "cuda:0"
N_CASES = 48


def draw_case(i):
    r = np.random.default_rng(1000 + i)
    decode = bool(r.random() < 0.4)
    L = int(r.integers(1, 65)) if decode else int(r.integers(1, 301))
    S = int(r.integers(1, 601))
    Hkv = int(r.integers(1, 4))
    G = int(r.choice([1, 2, 3, 5, 8]))
    mode = r.random()
    if mode < 0.2:
        off, W = NO_CAUSAL, 0
    else:
        off = int(r.choice([0, max(0, S - L), int(r.integers(0, S + 40))]))
        W = int(r.integers(1, S + 2)) if r.random() < 0.35 else 0
    return dict(B=int(r.integers(1, 4)), Hq=Hkv * G, Hkv=Hkv, D=int(r.choice([64, 128])), L=L, S=S,
                causal_offset=off, window=W, amp=1.0,
                key_padding=(1, S) if r.random() < 0.3 else None,
                sinks=bool(r.random() < 0.3),
                softcap=float(r.choice([0.0, 0.0, 5.0, 30.0])),
                entry="decode" if decode else "prefill")


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    c = draw_case(i)
    print(f"random shape case {i}: {c}", flush=True)
    x = make_inputs(c, seed=2000 + i)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    mask = torch.from_numpy(x["key_mask"]).to(DEV) if x["key_mask"] is not None else None
    sinks = torch.from_numpy(x["sinks"]).to(DEV) if x["sinks"] is not None else None
    off, W = x["causal_offset"], x["window"]
    kw = dict(scale=float(x["scale"]), causal=off >= 0, causal_offset=off if off >= 0 else None, window=W,
              key_mask=mask, softcap=c["softcap"], sinks=sinks)
    if c["entry"] == "decode":
        out = pfa.prefill_attn_gqa_decode(q, k, v, **kw)
    else:
        out = pfa.prefill_attn_gqa(q, k, v, **kw)
        out_ns = pfa.prefill_attn_gqa(q, k, v, no_skip=True, **kw)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], off, W, x["key_mask"], workers=16,
                      softcap=c["softcap"], sinks=x["sinks"])
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    rms_ref = float(np.sqrt(np.mean(ref ** 2)))
    rms_err = float(np.sqrt(np.mean(err ** 2)))
    msg = f"case {i} {c}: max_abs={err.max():.3e} rms_err={rms_err:.3e} rms_ref={rms_ref:.3e} bad={int(bad.sum())}"
    assert not bad.any(), msg
    if rms_ref > 0:
        assert rms_err <= RMS_RATIO * rms_ref, msg
    empty = ~np.any(np.abs(ref) > 0, axis=-1)
    assert np.all(got[empty] == 0.0), msg
    if c["entry"] == "prefill":
        assert torch.equal(out.view(torch.int16), out_ns.view(torch.int16)), f"skip != no-skip: {msg}"


# ---- packed variable-length batches ----

N_VARLEN = 24


def check(got, ref, msg):
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    rms_ref = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    rms_err = float(np.sqrt(np.mean(err ** 2))) if ref.size else 0.0
    full = f"{msg}: max_abs={err.max(initial=0):.3e} rms_err={rms_err:.3e} rms_ref={rms_ref:.3e} bad={int(bad.sum())}"
    assert not bad.any(), full
    if rms_ref > 0:
        assert rms_err <= RMS_RATIO * rms_ref, full
    empty = ~np.any(np.abs(ref) > 0, axis=-1)
    assert np.all(got[empty] == 0.0), full


def draw_varlen(i):
    r = np.random.default_rng(3000 + i)
    n = int(r.integers(1, 7))
    causal = bool(r.random() < 0.75)
    lq = r.integers(0, 301, size=n)
    lq[int(r.integers(0, n))] = max(1, int(lq.max()))  # at least one row in the batch
    lk = lq + r.integers(0, 301, size=n) if causal else r.integers(0, 401, size=n)
    lk[int(r.integers(0, n))] = max(1, int(lk.max()))  # at least one key in the batch
    Hkv = int(r.integers(1, 3))
    return dict(n_seq=n, Hq=Hkv * int(r.choice([1, 2, 4])), Hkv=Hkv, D=int(r.choice([64, 128])), lq=(0, 0),
                prefix=(0, 0), causal=causal, window=int(r.integers(1, 400)) if causal and r.random() < 0.35 else 0,
                lengths_q=[int(t) for t in lq], lengths_k=[int(t) for t in lk],
                softcap=float(r.choice([0.0, 0.0, 20.0])), sinks=bool(r.random() < 0.3))


@pytest.mark.parametrize("i", range(N_VARLEN))
def test_random_varlen(i):
    from oracle.varlen import oracle_varlen
    from workloads import make_varlen_inputs

    c = draw_varlen(i)
    print(f"random varlen case {i}: {c}", flush=True)
    x = make_varlen_inputs({k: c[k] for k in ("n_seq", "Hq", "Hkv", "D", "lq", "prefix", "causal", "window")},
                           seed=4000 + i, lengths_q=c["lengths_q"], lengths_k=c["lengths_k"])
    sinks = np.random.default_rng(5000 + i).standard_normal(c["Hq"], dtype=np.float32) if c["sinks"] else None
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    cq = torch.from_numpy(x["cu_q"]).to(DEV)
    ck = torch.from_numpy(x["cu_k"]).to(DEV)
    kw = dict(scale=float(x["scale"]), causal=x["causal"], window=x["window"], softcap=c["softcap"],
              sinks=torch.from_numpy(sinks).to(DEV) if sinks is not None else None)
    out = pfa.prefill_attn_gqa_varlen(q, k, v, cq, ck, x["max_seqlen_q"], **kw)
    out_ns = pfa.prefill_attn_gqa_varlen(q, k, v, cq, ck, x["max_seqlen_q"], no_skip=True, **kw)
    torch.cuda.synchronize()
    ref = oracle_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], x["scale"], x["causal"], x["window"],
                        softcap=c["softcap"], sinks=sinks)
    check(out.double().cpu().numpy(), ref, f"varlen case {i} {c}")
    assert torch.equal(out.view(torch.int16), out_ns.view(torch.int16)), f"varlen case {i}: skip != no-skip"


# ---- rotating cache ----

N_RING = 24


def draw_ring(i):
    r = np.random.default_rng(6000 + i)
    L = int(r.integers(1, 201))
    pos0 = int(r.choice([0, int(r.integers(0, 200)), int(r.integers(0, 3001))]))
    W = int(r.integers(1, 601)) if r.random() < 0.6 else 0
    need = min(W - 1 + L, pos0 + L) if W > 0 else pos0 + L
    ring = max(64, need + int(r.choice([0, 0, int(r.integers(1, 100))])))
    Hkv = int(r.integers(1, 3))
    return dict(B=int(r.integers(1, 3)), Hq=Hkv * int(r.choice([1, 2, 4])), Hkv=Hkv, D=int(r.choice([64, 128])),
                L=L, pos0=pos0, W=W, ring=ring, softcap=float(r.choice([0.0, 0.0, 20.0])),
                sinks=bool(r.random() < 0.3))


@pytest.mark.parametrize("i", range(N_RING))
def test_random_ring(i):
    from workloads import random_bits

    c = draw_ring(i)
    print(f"random ring case {i}: {c}", flush=True)
    B, Hq, Hkv, D, L, pos0, W, ring = (c[k] for k in ("B", "Hq", "Hkv", "D", "L", "pos0", "W", "ring"))
    rng = np.random.default_rng(7000 + i)
    q = random_bits(rng, (B, Hq, L, D))
    k_log = random_bits(rng, (B, Hkv, pos0 + L, D))
    v_log = random_bits(rng, (B, Hkv, pos0 + L, D))
    k_ring = random_bits(rng, (B, Hkv, ring, D), amp=4.0)  # stale slots: values no row may see
    v_ring = random_bits(rng, (B, Hkv, ring, D), amp=4.0)
    for p in range(max(0, pos0 - ring), pos0):
        k_ring[:, :, p % ring] = k_log[:, :, p]
        v_ring[:, :, p % ring] = v_log[:, :, p]
    sinks = rng.standard_normal(Hq, dtype=np.float32) if c["sinks"] else None
    scale = np.float32(1.0 / np.sqrt(np.float32(D)))
    opts = dict(softcap=c["softcap"], sinks=torch.from_numpy(sinks).to(DEV) if sinks is not None else None)
    qd = dev_bf16(q)
    out = pfa.prefill_attn_gqa_ring(qd, dev_bf16(k_log[:, :, pos0:]), dev_bf16(v_log[:, :, pos0:]), dev_bf16(k_ring),
                                    dev_bf16(v_ring), pos0, scale=float(scale), window=W, **opts)
    dense = pfa.prefill_attn_gqa(qd, dev_bf16(k_log), dev_bf16(v_log), scale=float(scale), causal_offset=pos0,
                                 window=W, **opts)
    torch.cuda.synchronize()
    ref = oracle_sdpa(q, k_log, v_log, scale, pos0, W, None, workers=16, softcap=c["softcap"], sinks=sinks)
    check(out.double().cpu().numpy(), ref, f"ring case {i} {c}")
    assert torch.equal(out.view(torch.int16), dense.view(torch.int16)), f"ring case {i}: ring != dense on the logical keys"


# ---- dense-only options: additive bias, block bitmap ----

N_OPT = 24


def draw_opt(i):
    r = np.random.default_rng(8000 + i)
    L, S = int(r.integers(1, 301)), int(r.integers(1, 601))
    Hkv = int(r.integers(1, 3))
    off = NO_CAUSAL if r.random() < 0.2 else int(r.choice([0, max(0, S - L), int(r.integers(0, S + 40))]))
    W = int(r.integers(1, S + 2)) if off >= 0 and r.random() < 0.35 else 0
    return dict(B=int(r.integers(1, 3)), Hq=Hkv * int(r.choice([1, 2, 4])), Hkv=Hkv, D=int(r.choice([64, 128])),
                L=L, S=S, causal_offset=off, window=W, amp=1.0, key_padding=None,
                softcap=float(r.choice([0.0, 0.0, 20.0])), sinks=bool(r.random() < 0.3),
                kind="bias" if i % 2 == 0 else "sel",
                bias_shape=int(r.integers(0, 5)), sel_shape=int(r.integers(0, 3)),
                block_q=int(r.choice([32, 64, 96, 128, 256])), block_k=int(r.choice([64, 128, 192, 320])),
                density=float(r.uniform(0.2, 0.8)))


@pytest.mark.parametrize("i", range(N_OPT))
def test_random_bias_and_bitmap(i):
    c = draw_opt(i)
    print(f"random option case {i}: {c}", flush=True)
    x = make_inputs({k: c[k] for k in ("B", "Hq", "Hkv", "D", "L", "S", "causal_offset", "window", "amp",
                                       "key_padding", "sinks")}, seed=9000 + i)
    B, Hq, L, S = c["B"], c["Hq"], c["L"], c["S"]
    r = np.random.default_rng(9500 + i)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    sinks = x["sinks"]
    off, W = x["causal_offset"], x["window"]
    kw = dict(scale=float(x["scale"]), causal=off >= 0, causal_offset=off if off >= 0 else None, window=W,
              softcap=c["softcap"], sinks=torch.from_numpy(sinks).to(DEV) if sinks is not None else None)
    ref_kw = {}
    if c["kind"] == "bias":
        # one of [L,S], [1,Hq,L,S], [B,1,L,S], [B,Hq,L,S], [1,1,1,S]; about 10 % of entries -inf; the key
        # dimension padded to a multiple of 4 elements (the row stride the library requires)
        shape = [(1, 1, L, S), (1, Hq, L, S), (B, 1, L, S), (B, Hq, L, S), (1, 1, 1, S)][c["bias_shape"]]
        vals = (r.standard_normal(shape, dtype=np.float32) * np.float32(2.0))
        vals[r.random(shape) < 0.1] = -np.inf
        S4 = -(-S // 4) * 4
        buf = torch.zeros(shape[:3] + (S4,), dtype=torch.float32, device=DEV)
        buf[..., :S] = torch.from_numpy(vals).to(DEV)
        kw["bias"] = buf[..., :S] if c["bias_shape"] != 0 else buf[0, 0, :, :S]
        ref_kw["bias"] = vals
    else:
        bq, bk = c["block_q"], c["block_k"]
        nqb, nkb = -(-L // bq), -(-S // bk)
        shape = [(nqb, nkb), (Hq, nqb, nkb), (B, Hq, nqb, nkb)][c["sel_shape"]]
        sel = (r.random(shape) < c["density"]).astype(np.uint8)
        kw.update(block_sel=torch.from_numpy(sel).to(DEV), block_q=bq, block_k=bk)
        ref_kw.update(block_sel=sel, block_q=bq, block_k=bk)
    out = pfa.prefill_attn_gqa(q, k, v, **kw)
    out_ns = pfa.prefill_attn_gqa(q, k, v, no_skip=True, **kw)
    torch.cuda.synchronize()
    ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], off, W, None, workers=16, softcap=c["softcap"],
                      sinks=sinks, **ref_kw)
    check(out.double().cpu().numpy(), ref, f"option case {i} {c}")
    assert torch.equal(out.view(torch.int16), out_ns.view(torch.int16)), f"option case {i}: skip != no-skip"
