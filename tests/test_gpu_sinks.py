"""GPU parity of attention sinks (one logit per query head that joins every row's softmax as an
extra term with no value; mlx-lm sliding-window prefill PR, "Correctness", lists attention sinks
among its cases) on the prefill and decode entry points, against the fp64 CPU oracle; skip ==
no-skip bit for bit with sinks; -inf sinks are no sinks, bit for bit.

Tolerance as in test_gpu_parity.py (atol = rtol = 2e-2 elementwise, rms ratio <= 1e-2).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import prefill_attention_amd as pfa  # noqa: E402
from oracle import oracle_sdpa  # noqa: E402
from workloads import make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

ATOL = RTOL = 2e-2
RMS_RATIO = 1e-2
DEV = "cuda:0"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def check_close(got, ref, what=""):
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    rms_ref = float(np.sqrt(np.mean(ref ** 2)))
    rms_err = float(np.sqrt(np.mean(err ** 2)))
    msg = f"{what}: max_abs={err.max():.3e} rms_err={rms_err:.3e} rms_ref={rms_ref:.3e} bad={int(bad.sum())}"
    assert not bad.any(), msg
    if rms_ref > 0:
        assert rms_err <= RMS_RATIO * rms_ref, msg


def sink_logits(rng, Hq):
    """N(0, 2) logits per head, with one head at -inf (no sink) and one at 6 (a dominant sink)."""
    s = (rng.standard_normal(Hq) * 2.0).astype(np.float32)
    s[0] = -np.inf
    if Hq > 2:
        s[2] = 6.0
    return s


# (name, B, Hq, Hkv, D, L, S, causal_offset, window, key padding, softcap, bias)
CASES = [
    ("witness", 1, 4, 2, 128, 33, 47, 14, 0, None, 0.0, False),
    ("causal_l300_s900", 1, 8, 2, 128, 300, 900, 600, 0, None, 0.0, False),
    ("window_d64", 1, 8, 4, 64, 400, 1000, 600, 200, None, 0.0, False),
    ("keymask_bidir", 2, 4, 2, 128, 100, 300, -1, 0, (1, 300), 0.0, False),
    ("softcap_bias", 1, 4, 2, 128, 257, 700, 443, 0, None, 4.0, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sinks_prefill_parity_and_skip_identity(case):
    name, B, Hq, Hkv, D, L, S, off, W, kp, cap, with_bias = case
    x = make_inputs(dict(B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, S=S, causal_offset=off, window=W, amp=1.0,
                         key_padding=kp), seed=81)
    rng = np.random.default_rng(82)
    sinks = sink_logits(rng, Hq)
    bias = None
    bt = None
    if with_bias:
        S4 = (S + 3) // 4 * 4
        bias = (rng.standard_normal((L, S)) * 2.0).astype(np.float32)
        padded = np.zeros((L, S4), dtype=np.float32)
        padded[:, :S] = bias
        bt = torch.from_numpy(padded).to(DEV)[:, :S]
    print(f"sinks prefill {name}", flush=True)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    mask = torch.from_numpy(x["key_mask"]).to(DEV) if x["key_mask"] is not None else None
    st = torch.from_numpy(sinks).to(DEV)
    kw = dict(scale=float(x["scale"]), causal=off >= 0, causal_offset=off if off >= 0 else None, window=W,
              key_mask=mask, softcap=cap, bias=bt)
    out = pfa.prefill_attn_gqa(q, k, v, sinks=st, **kw)
    out_ns = pfa.prefill_attn_gqa(q, k, v, sinks=st, no_skip=True, **kw)
    plain = pfa.prefill_attn_gqa(q, k, v, **kw)
    none = pfa.prefill_attn_gqa(q, k, v, sinks=torch.full_like(st, -float("inf")), **kw)
    torch.cuda.synchronize()
    ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], off, W, x["key_mask"], workers=16, softcap=cap,
                      bias=None if bias is None else bias.astype(np.float64), sinks=sinks.astype(np.float64))
    check_close(out.double().cpu().numpy(), ref, name)
    assert torch.equal(out.view(torch.int16), out_ns.view(torch.int16))
    assert torch.equal(plain.view(torch.int16), none.view(torch.int16))
    # head 0 has no sink: its rows equal the plain call's bit for bit
    assert torch.equal(out[:, 0].view(torch.int16), plain[:, 0].view(torch.int16))


# (name, B, Hq, Hkv, D, L, S, causal_offset, key padding, softcap)
DECODE_CASES = [
    ("l1_s9000", 1, 32, 8, 128, 1, 9000, 8999, None, 0.0),
    ("l8_s3000_d64", 2, 8, 2, 64, 8, 3000, 2992, None, 0.0),
    ("l4_keymask_cap", 2, 8, 4, 128, 4, 2000, 1996, (1, 2000), 3.0),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_sinks_decode_parity(case):
    name, B, Hq, Hkv, D, L, S, off, kp, cap = case
    x = make_inputs(dict(B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, S=S, causal_offset=off, window=0, amp=1.0,
                         key_padding=kp), seed=83)
    sinks = sink_logits(np.random.default_rng(84), Hq)
    print(f"sinks decode {name}", flush=True)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    mask = torch.from_numpy(x["key_mask"]).to(DEV) if x["key_mask"] is not None else None
    kw = dict(scale=float(x["scale"]), causal_offset=off, key_mask=mask, softcap=cap)
    out = pfa.prefill_attn_gqa_decode(q, k, v, sinks=torch.from_numpy(sinks).to(DEV), **kw)
    plain = pfa.prefill_attn_gqa_decode(q, k, v, **kw)
    torch.cuda.synchronize()
    ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], off, 0, x["key_mask"], workers=16, softcap=cap,
                      sinks=sinks.astype(np.float64))
    check_close(out.double().cpu().numpy(), ref, name)
    assert torch.equal(out[:, 0].view(torch.int16), plain[:, 0].view(torch.int16))
