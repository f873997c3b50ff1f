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
