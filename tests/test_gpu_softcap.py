"""GPU parity of logit soft-capping (brotensor flash_attention_decode, attn_softcap: after the scale
and before the masks, each score s becomes cap * tanh(s / cap)) on the prefill and decode entry
points, against the fp64 CPU oracle; skip == no-skip bit for bit with the cap on.

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


# (name, B, Hq, Hkv, D, L, S, causal_offset, window, key padding, amp, cap)
CASES = [
    ("witness_cap2", 1, 4, 2, 128, 33, 47, 14, 0, None, 1.0, 2.0),
    ("causal_l300_s900_cap5", 1, 8, 2, 128, 300, 900, 600, 0, None, 2.0, 5.0),
    ("window_d64_cap50", 1, 8, 4, 64, 400, 1000, 600, 200, None, 4.0, 50.0),
    ("keymask_bidir_cap1", 2, 4, 2, 128, 100, 300, -1, 0, (1, 300), 1.0, 1.0),
]


def inputs(case):
    name, B, Hq, Hkv, D, L, S, off, W, kp, amp, cap = case
    return make_inputs(dict(B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, S=S, causal_offset=off, window=W, amp=amp,
                            key_padding=kp), seed=51), cap


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_softcap_prefill_parity_and_skip_identity(case):
    x, cap = inputs(case)
    print(f"softcap prefill {case[0]}", flush=True)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    mask = torch.from_numpy(x["key_mask"]).to(DEV) if x["key_mask"] is not None else None
    off = x["causal_offset"]
    kw = dict(scale=float(x["scale"]), causal=off >= 0, causal_offset=off if off >= 0 else None, window=x["window"],
              key_mask=mask, softcap=cap)
    out = pfa.prefill_attn_gqa(q, k, v, **kw)
    out_ns = pfa.prefill_attn_gqa(q, k, v, no_skip=True, **kw)
    torch.cuda.synchronize()
    ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], off, x["window"], x["key_mask"], workers=16, softcap=cap)
    check_close(out.double().cpu().numpy(), ref, case[0])
    assert torch.equal(out.view(torch.int16), out_ns.view(torch.int16))
    # the cap changes the result where it bites (guards against the cap being ignored)
    plain = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], off, x["window"], x["key_mask"], workers=16)
    if cap <= 5.0:
        assert np.abs(plain - ref).max() > 0.05


@pytest.mark.parametrize("cap", [3.0, 50.0])
def test_softcap_decode_parity(cap):
    x = make_inputs(dict(B=1, Hq=32, Hkv=8, D=128, L=2, S=5000, causal_offset=4998, window=0, amp=2.0,
                         key_padding=None), seed=52)
    print(f"softcap decode cap={cap}", flush=True)
    out = pfa.prefill_attn_gqa_decode(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), scale=float(x["scale"]),
                                      causal_offset=4998, softcap=cap)
    torch.cuda.synchronize()
    ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], 4998, 0, None, workers=16, softcap=cap)
    check_close(out.double().cpu().numpy(), ref, f"decode cap={cap}")
