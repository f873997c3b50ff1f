"""GPU parity of the variant workloads at their full sizes, launched the way the benchmark launches
them (same entry point, arguments and preallocated buffers): the soft-capped and biased chunks,
attention sinks, the block bitmap, the rotating cache and the short-query (decode) shapes. Every
output element is checked against the fp64 CPU oracle (a few seconds of oracle time each on the
host's cores); the prefill variants also check skip == no-skip bit for bit at full size.

Tolerance as in test_gpu_parity.py (atol = rtol = 2e-2 elementwise, rms ratio <= 1e-2).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import prefill_attention_amd as pfa  # noqa: E402
from oracle import host_workers, oracle_sdpa  # noqa: E402
from workloads import CONFIGS, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

ATOL = RTOL = 2e-2
RMS_RATIO = 1e-2
DEV = "cuda:0"
WORKERS = max(1, min(16, host_workers()))


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
    return msg


def run_workload(name, no_skip=False):
    """Launch the workload as the benchmark does; returns (inputs, output tensor)."""
    c = CONFIGS[name]
    x = make_inputs(name, seed=0)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    out = torch.empty_like(q)
    off = x["causal_offset"]
    if c.get("entry") == "ring":
        pos0, ring = off, c["ring"]
        k_new, v_new = k[:, :, pos0:].contiguous(), v[:, :, pos0:].contiguous()
        k_ring = torch.zeros(c["B"], c["Hkv"], ring, c["D"], dtype=torch.bfloat16, device=DEV)
        v_ring = torch.zeros_like(k_ring)
        for p0 in range(max(0, pos0 - ring), pos0):
            k_ring[:, :, p0 % ring] = k[:, :, p0]
            v_ring[:, :, p0 % ring] = v[:, :, p0]
        pfa.prefill_attn_gqa_ring(q, k_new, v_new, k_ring, v_ring, pos0, scale=float(x["scale"]),
                                  window=c["window"], out=out)
        torch.cuda.synchronize()
        return x, out
    kw = dict(scale=float(x["scale"]), causal=off >= 0, causal_offset=off if off >= 0 else None,
              window=x["window"], out=out)
    if c.get("softcap"):
        kw["softcap"] = float(c["softcap"])
    if x.get("bias") is not None:
        kw["bias"] = torch.from_numpy(x["bias"]).to(DEV)
    if x.get("sinks") is not None:
        kw["sinks"] = torch.from_numpy(x["sinks"]).to(DEV)
    if x.get("block_sel") is not None:
        kw.update(block_sel=torch.from_numpy(x["block_sel"]).to(DEV), block_q=x["block_q"], block_k=x["block_k"])
    if c.get("entry") == "decode":
        kw["workspace"] = torch.empty(pfa.decode_workspace_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["S"], c["D"]),
                                      dtype=torch.uint8, device=DEV)
        pfa.prefill_attn_gqa_decode(q, k, v, **kw)
    else:
        pfa.prefill_attn_gqa(q, k, v, no_skip=no_skip, **kw)
    torch.cuda.synchronize()
    return x, out


PREFILL = ["long_ctx_32k_softcap50", "mid_ctx_8k_bias", "long_ctx_32k_sinks", "long_ctx_32k_sel"]
OTHER = ["ring_w1024_l2048", "decode_l1_32k", "decode_l8_8k", "decode_b8_l1_4k"]


@pytest.mark.parametrize("name", PREFILL + OTHER)
def test_full_size_full_oracle(name):
    print(f"[parity] {name} (full size, every output element)", flush=True)
    x, out = run_workload(name)
    got = out.double().cpu().numpy()
    del out
    sel = x.get("block_sel")
    ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], x["causal_offset"], x["window"], x["key_mask"],
                      workers=WORKERS, softcap=float(CONFIGS[name].get("softcap", 0.0)),
                      bias=None if x.get("bias") is None else x["bias"].astype(np.float64),
                      sinks=None if x.get("sinks") is None else x["sinks"].astype(np.float64),
                      block_sel=None if sel is None else sel[None], block_q=x["block_q"] or 0,
                      block_k=x["block_k"] or 0)
    print(check_close(got, ref, name), flush=True)


@pytest.mark.parametrize("name", PREFILL)
def test_full_size_skip_identity(name):
    print(f"[bitwise] {name} (full size)", flush=True)
    _, out = run_workload(name)
    _, out_ns = run_workload(name, no_skip=True)
    assert torch.equal(out.view(torch.int16), out_ns.view(torch.int16))
