"""The allocation-free decode entry point (prefill_attn_gqa_decode_noalloc) against the decode entry
point with a caller workspace (prefill_attn_gqa_decode), through the C ABI: the same kernels and
split plan, so the outputs must be equal bit for bit, and both within the oracle tolerance
(|O_gpu - O_ref| <= 2e-2 + 2e-2 |O_ref| elementwise, rms(err)/rms(ref) <= 1e-2). Two calls in a row,
the second on a smaller shape, share the library's scratch array; a shape too large for the array is
refused on the host.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import prefill_attention_amd as pfa  # noqa: E402
from oracle import host_workers, oracle_sdpa  # noqa: E402
from workloads import make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

ATOL = RTOL = 2e-2
RMS_RATIO = 1e-2
DEV = "cuda:0"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def check_close(got, ref, what):
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    rms_ref = float(np.sqrt(np.mean(ref ** 2)))
    rms_err = float(np.sqrt(np.mean(err ** 2)))
    msg = f"{what}: max_abs={err.max():.3e} rms_err={rms_err:.3e} rms_ref={rms_ref:.3e} bad={int(bad.sum())}"
    assert not bad.any(), msg
    if rms_ref > 0:
        assert rms_err <= RMS_RATIO * rms_ref, msg


def both(x, softcap=0.0, sinks=None):
    """(no-alloc output, caller-workspace output) for the inputs x, both through the C ABI."""
    B, Hq, L, D = x["q"].shape
    Hkv, S = x["k"].shape[1], x["k"].shape[2]
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    mask = torch.from_numpy(x["key_mask"]).to(DEV) if x.get("key_mask") is not None else None
    sk = torch.from_numpy(sinks).to(DEV) if sinks is not None else None
    o_na = torch.empty_like(q)
    o_ws = torch.empty_like(q)
    ws = torch.empty(max(16, pfa.decode_workspace_bytes(B, Hq, Hkv, L, S, D)), dtype=torch.uint8, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), B, Hq, Hkv, L, S, D, float(x["scale"]), x["causal_offset"],
            x["window"], None if mask is None else mask.data_ptr())
    rc = pfa.prefill_attn_gqa_decode_noalloc_raw(*args, o_na.data_ptr(), st, softcap, 0,
                                                 None if sk is None else sk.data_ptr())
    assert rc == 0, pfa.status_str(rc)
    torch.cuda.synchronize()
    rc = pfa.prefill_attn_gqa_decode_raw(*args, o_ws.data_ptr(), ws.data_ptr(), ws.numel(), st, softcap, 0,
                                         None if sk is None else sk.data_ptr())
    assert rc == 0, pfa.status_str(rc)
    torch.cuda.synchronize()
    return o_na, o_ws


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    # first a large shape (56 rows per KV head, 14 MiB of partials), then a smaller one with a key
    # mask, a window, a soft-cap and sinks: the second call must not see the first call's partials
    big = make_inputs("decode_l8_8k", seed=0)
    small = make_inputs(dict(B=2, Hq=8, Hkv=2, D=64, L=3, S=700, causal_offset=697, window=200, amp=1.0,
                             key_padding=(300, 700)), seed=41)
    sinks = np.random.default_rng(42).standard_normal(8).astype(np.float32)
    workers = max(1, min(16, host_workers()))
    for name, x, softcap, sk in (("decode_l8_8k", big, 0.0, None), ("small_masked_window", small, 30.0, sinks)):
        print(f"noalloc decode {name}", flush=True)
        o_na, o_ws = both(x, softcap, sk)
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), name
        ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], x["causal_offset"], x["window"], x["key_mask"],
                          workers=workers, softcap=softcap, sinks=None if sk is None else sk.astype(np.float64))
        check_close(o_na.double().cpu().numpy(), ref, name)


def test_noalloc_refuses_shapes_beyond_the_scratch_array():
    B, Hq, Hkv, L, S, D = 64, 64, 8, 16, 131072, 128
    assert pfa.decode_workspace_bytes(B, Hq, Hkv, L, S, D) > pfa.DECODE_SCRATCH_BYTES
    q = torch.empty(1, dtype=torch.bfloat16, device=DEV)
    # the size check runs on the host before any device address is used
    rc = pfa.prefill_attn_gqa_decode_noalloc_raw(q.data_ptr(), q.data_ptr() + 2 ** 36, q.data_ptr() + 2 ** 37, B, Hq,
                                                 Hkv, L, S, D, 0.088, S - L, 0, None, q.data_ptr() + 2 ** 38, None)
    assert rc == 11
