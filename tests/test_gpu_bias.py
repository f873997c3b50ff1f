"""GPU parity of the additive bias (tiny-llm Week 2 Day 5 Task 2: a broadcastable additive array
mask applied before the online-softmax update) on the prefill entry point, against the fp64 CPU
oracle; skip == no-skip bit for bit with a bias.

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


# (name, B, Hq, Hkv, D, L, S, causal_offset, window, bias shape, -inf fraction, softcap)
CASES = [
    ("ls_broadcast_causal", 1, 8, 2, 128, 300, 900, 600, 0, "LS", 0.0, 0.0),
    ("per_head_bidir", 2, 4, 2, 128, 130, 260, -1, 0, "BHLS", 0.0, 0.0),
    ("neg_inf_entries", 1, 4, 4, 128, 200, 333, 133, 0, "LS", 0.3, 0.0),
    ("d64_window", 1, 8, 4, 64, 400, 1000, 600, 200, "B1LS", 0.0, 0.0),
    ("with_softcap", 1, 4, 2, 128, 257, 700, 443, 0, "LS", 0.1, 4.0),
]


def make_bias(rng, kind, B, Hq, L, S, neg):
    shape = {"LS": (L, S), "BHLS": (B, Hq, L, S), "B1LS": (B, 1, L, S)}[kind]
    b = (rng.standard_normal(shape) * 2.0).astype(np.float32)
    if neg > 0:
        b[rng.random(shape) < neg] = -np.inf
    return b


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bias_parity_and_skip_identity(case):
    name, B, Hq, Hkv, D, L, S, off, W, kind, neg, cap = case
    x = make_inputs(dict(B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, S=S, causal_offset=off, window=W, amp=1.0, key_padding=None),
                    seed=61)
    bias = make_bias(np.random.default_rng(62), kind, B, Hq, L, S, neg)
    # keep the key dimension a multiple of 4 elements apart (16-byte rows): pad the row stride
    S4 = (S + 3) // 4 * 4
    padded = np.zeros(bias.shape[:-1] + (S4,), dtype=np.float32)
    padded[..., :S] = bias
    bt = torch.from_numpy(padded).to(DEV)[..., :S]
    print(f"bias {name}", flush=True)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    kw = dict(scale=float(x["scale"]), causal=off >= 0, causal_offset=off if off >= 0 else None, window=W,
              bias=bt, softcap=cap)
    out = pfa.prefill_attn_gqa(q, k, v, **kw)
    out_ns = pfa.prefill_attn_gqa(q, k, v, no_skip=True, **kw)
    torch.cuda.synchronize()
    ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], off, W, None, workers=16, softcap=cap,
                      bias=bias.astype(np.float64))
    check_close(out.double().cpu().numpy(), ref, name)
    assert torch.equal(out.view(torch.int16), out_ns.view(torch.int16))
    # rows the bias masks completely are exact zeros
    empty = ~np.any(np.abs(ref) > 0, axis=-1)
    assert np.all(out.double().cpu().numpy()[empty] == 0.0)


def test_bias_unaligned_rows_rejected():
    x = make_inputs(dict(B=1, Hq=4, Hkv=2, D=128, L=16, S=30, causal_offset=14, window=0, amp=1.0,
                         key_padding=None), seed=63)
    bt = torch.zeros(16, 30, dtype=torch.float32, device=DEV)  # row stride 30: not a multiple of 4
    with pytest.raises(pfa.PfaError, match="ALIGN"):
        pfa.prefill_attn_gqa(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), causal_offset=14, bias=bt)
