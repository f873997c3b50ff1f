"""GPU tests of the rotating-cache entry point: the chunk's keys are appended to their ring slots
and the attention reads every key through the slot map. Checked against the fp64 CPU oracle on the
logical keys (history followed by the chunk), bit for bit against the dense entry point on those
logical keys, and the ring contents after the call bit for bit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import prefill_attention_amd as pfa  # noqa: E402
from oracle import oracle_sdpa, oracle_selected_rows  # noqa: E402
from workloads import random_bits  # noqa: E402

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


def make_case(B, Hq, Hkv, D, L, pos0, ring, W, seed):
    rng = np.random.default_rng(seed)
    q = random_bits(rng, (B, Hq, L, D))
    k_hist = random_bits(rng, (B, Hkv, pos0, D))
    v_hist = random_bits(rng, (B, Hkv, pos0, D))
    k_new = random_bits(rng, (B, Hkv, L, D))
    v_new = random_bits(rng, (B, Hkv, L, D))
    k_ring = random_bits(rng, (B, Hkv, ring, D), amp=4.0)  # stale slots: values no row may see
    v_ring = random_bits(rng, (B, Hkv, ring, D), amp=4.0)
    for p in range(max(0, pos0 - ring), pos0):
        k_ring[:, :, p % ring] = k_hist[:, :, p]
        v_ring[:, :, p % ring] = v_hist[:, :, p]
    k_log = np.concatenate([k_hist, k_new], axis=2)
    v_log = np.concatenate([v_hist, v_new], axis=2)
    return dict(q=q, k_new=k_new, v_new=v_new, k_ring=k_ring, v_ring=v_ring, k_log=k_log, v_log=v_log,
                scale=np.float32(1.0 / np.sqrt(np.float32(D))), pos0=pos0, W=W, L=L, ring=ring)


# (name, B, Hq, Hkv, D, L, pos0, ring, window, full oracle)
CASES = [
    ("decode_chunk_ring_w_plus_64", 2, 8, 2, 128, 16, 7777, 1088, 1024, True),
    ("chunk2048_w1024", 1, 8, 2, 128, 2048, 5000, 3072, 1024, False),
    ("d64_full_causal", 1, 4, 4, 64, 300, 100, 448, 0, True),
    ("fresh_cache", 1, 4, 2, 128, 130, 0, 192, 0, True),
    ("ring_not_multiple_of_64", 1, 4, 2, 128, 50, 3000, 1100, 1024, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ring_prefill(case):
    name, B, Hq, Hkv, D, L, pos0, ring, W, full = case
    x = make_case(B, Hq, Hkv, D, L, pos0, ring, W, seed=41)
    print(f"ring {name}", flush=True)
    q, kn, vn = dev_bf16(x["q"]), dev_bf16(x["k_new"]), dev_bf16(x["v_new"])
    kr, vr = dev_bf16(x["k_ring"]), dev_bf16(x["v_ring"])
    out = pfa.prefill_attn_gqa_ring(q, kn, vn, kr, vr, pos0, scale=float(x["scale"]), window=W)
    torch.cuda.synchronize()
    # ring contents: the chunk's rows in their slots, every other slot untouched
    kr_h = kr.view(torch.int16).cpu().numpy().view(np.uint16)
    vr_h = vr.view(torch.int16).cpu().numpy().view(np.uint16)
    want_k, want_v = x["k_ring"].copy(), x["v_ring"].copy()
    for i in range(L):
        want_k[:, :, (pos0 + i) % ring] = x["k_new"][:, :, i]
        want_v[:, :, (pos0 + i) % ring] = x["v_new"][:, :, i]
    assert np.array_equal(kr_h, want_k) and np.array_equal(vr_h, want_v)
    # bit-identical to the dense entry point on the logical keys
    dense = pfa.prefill_attn_gqa(q, dev_bf16(x["k_log"]), dev_bf16(x["v_log"]), scale=float(x["scale"]),
                                 causal_offset=pos0, window=W)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), dense.view(torch.int16))
    # against the oracle on the logical keys
    got = out.double().cpu().numpy()
    if full:
        ref = oracle_sdpa(x["q"], x["k_log"], x["v_log"], x["scale"], pos0, W, None, workers=16)
        check_close(got, ref, name)
    else:
        rng = np.random.default_rng(3)
        picks = [(0, int(h), int(i)) for h, i in zip(rng.integers(0, Hq, 24), rng.integers(0, L, 24))]
        picks += [(0, 0, 0), (0, Hq - 1, L - 1)]
        ref = oracle_selected_rows(x["q"], x["k_log"], x["v_log"], x["scale"], pos0, W, None, picks)
        check_close(np.array([got[b, h, i] for b, h, i in picks]), ref, name)


def test_ring_too_small_raises_and_touches_nothing():
    x = make_case(1, 4, 2, 128, 64, 2000, 1088, 1100, seed=42)  # needs 1100 - 1 + 64 slots
    kr = dev_bf16(x["k_ring"])
    before = kr.clone()
    with pytest.raises(pfa.PfaError, match="RING"):
        pfa.prefill_attn_gqa_ring(dev_bf16(x["q"]), dev_bf16(x["k_new"]), dev_bf16(x["v_new"]), kr,
                                  dev_bf16(x["v_ring"]), 2000, window=1100)
    torch.cuda.synchronize()
    assert torch.equal(kr.view(torch.int16), before.view(torch.int16))


@pytest.mark.parametrize("D,W", [(128, 1024), (64, 0)])
def test_ring_options(D, W):
    """Soft-cap and sinks through the rotating cache: bit-identical to the dense call with the same
    options on the logical keys, skip == no-skip bit for bit, and within tolerance of the oracle."""
    x = make_case(1, 8, 2, D, 200, 3000 if W else 400, 1280 if W else 640, W, seed=77)
    sinks = (np.random.default_rng(78).standard_normal(8) * 2.0).astype(np.float32)
    print(f"ring options D={D} W={W}", flush=True)
    st = torch.from_numpy(sinks).to(DEV)
    q = dev_bf16(x["q"])
    outs = []
    for no_skip in (False, True):
        kr, vr = dev_bf16(x["k_ring"]), dev_bf16(x["v_ring"])
        outs.append(pfa.prefill_attn_gqa_ring(q, dev_bf16(x["k_new"]), dev_bf16(x["v_new"]), kr, vr, x["pos0"],
                                              scale=float(x["scale"]), window=W, softcap=6.0, sinks=st,
                                              no_skip=no_skip))
    dense = pfa.prefill_attn_gqa(q, dev_bf16(x["k_log"]), dev_bf16(x["v_log"]), scale=float(x["scale"]),
                                 causal_offset=x["pos0"], window=W, softcap=6.0, sinks=st)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), dense.view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    ref = oracle_sdpa(x["q"], x["k_log"], x["v_log"], x["scale"], x["pos0"], W, None, workers=16, softcap=6.0,
                      sinks=sinks.astype(np.float64))
    check_close(outs[0].double().cpu().numpy(), ref, f"ring options D={D} W={W}")
