"""GPU parity at large logit magnitudes: inputs drawn as amp * N(0, 1) with amp 2 and 4, so that the
scaled scores reach tens of units and the softmax is sharply peaked. This guards the score and
exponent arithmetic (each score is formed in FP32 from the exact BF16 products and scaled in FP32;
no rounding of scaled operands back to BF16) on the prefill and decode entry points, against the fp64
CPU oracle, with the same tolerance as test_gpu_parity.py (atol = rtol = 2e-2 elementwise, rms ratio
<= 1e-2)."""
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


# (name, B, Hq, Hkv, D, L, S, causal_offset, window, key padding, entry)
CASES = [
    ("causal_d128", 1, 8, 2, 128, 300, 900, 600, 0, None, "prefill"),
    ("window_d64", 1, 8, 4, 64, 400, 1000, 600, 200, None, "prefill"),
    ("bidir_keymask", 2, 4, 2, 128, 200, 500, -1, 0, (1, 500), "prefill"),
    ("decode_l4", 2, 8, 2, 128, 4, 3000, 2996, 0, None, "decode"),
]


@pytest.mark.parametrize("amp", [2.0, 4.0])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_large_logits(case, amp):
    name, B, Hq, Hkv, D, L, S, off, W, kp, entry = case
    x = make_inputs(dict(B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, S=S, causal_offset=off, window=W, amp=amp,
                         key_padding=kp), seed=101)
    print(f"large logits {name} amp {amp}", flush=True)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    mask = torch.from_numpy(x["key_mask"]).to(DEV) if x["key_mask"] is not None else None
    kw = dict(scale=float(x["scale"]), causal=off >= 0, causal_offset=off if off >= 0 else None, window=W,
              key_mask=mask)
    fn = pfa.prefill_attn_gqa_decode if entry == "decode" else pfa.prefill_attn_gqa
    out = fn(q, k, v, **kw)
    torch.cuda.synchronize()
    ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], off, W, x["key_mask"], workers=16)
    check_close(out.double().cpu().numpy(), ref, f"{name} amp {amp}")
