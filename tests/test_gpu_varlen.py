"""GPU parity of the packed variable-length entry point against the fp64 CPU oracle, and its
bit-identity with the dense entry point sequence by sequence.

Tolerance as in test_gpu_parity.py: |O_gpu - O_ref| <= 2e-2 + 2e-2 |O_ref| elementwise (tiny-llm
Week 2 Day 5, Task 1) and rms(err)/rms(ref) <= 1e-2.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import prefill_attention_amd as pfa  # noqa: E402
from oracle import host_workers, oracle_varlen  # noqa: E402
from workloads import make_varlen_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

ATOL = RTOL = 2e-2
RMS_RATIO = 1e-2
DEV = "cuda:0"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def run_varlen(x, causal=None, window=None, out=None, cu_q=None, cu_k=None, max_q=None):
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    o = pfa.prefill_attn_gqa_varlen(
        q, k, v, dev_i32(x["cu_q"] if cu_q is None else cu_q), dev_i32(x["cu_k"] if cu_k is None else cu_k),
        x["max_seqlen_q"] if max_q is None else max_q, scale=float(x["scale"]),
        causal=x["causal"] if causal is None else causal, window=x["window"] if window is None else window,
        out=out)
    torch.cuda.synchronize()
    return o


def check_close(got, ref, what=""):
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    rms_ref = float(np.sqrt(np.mean(ref ** 2)))
    rms_err = float(np.sqrt(np.mean(err ** 2)))
    msg = f"{what}: max_abs={err.max():.3e} rms_err={rms_err:.3e} rms_ref={rms_ref:.3e} bad={int(bad.sum())}"
    assert not bad.any(), msg
    if rms_ref > 0:
        assert rms_err <= RMS_RATIO * rms_ref, msg


# ragged length sets: single rows, tails, several key tiles, a sequence without rows, one with
# more rows than keys, one longer than a 256-row workgroup, sequences with rows but no keys
LENGTHS = {
    "ragged": ([1, 33, 300, 0, 517, 64], [1, 40, 300, 10, 1100, 764]),
    "no_keys": ([3, 40, 7, 1], [0, 64, 0, 1]),
    "equal": ([5, 129, 256, 257, 90], [5, 129, 256, 257, 90]),
    "short_keys": ([200, 70], [37, 70]),
}


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("lengths", sorted(LENGTHS))
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 100)])
def test_varlen_parity(D, lengths, causal, window):
    lq, lk = LENGTHS[lengths]
    x = make_varlen_inputs("varlen_chunks_b5", seed=21, lengths_q=lq, lengths_k=lk, D=D)
    print(f"varlen parity D={D} {lengths} causal={causal} window={window}", flush=True)
    got = run_varlen(x, causal=causal, window=window).double().cpu().numpy()
    ref = oracle_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], x["scale"], causal, window)
    check_close(got, ref, f"D={D} {lengths} causal={causal} W={window}")
    # rows that see no key are exact zeros (every row of a sequence without keys)
    for b in range(len(lq)):
        s0 = int(x["cu_q"][b])
        if lk[b] == 0:
            assert torch.count_nonzero(torch.from_numpy(got[s0:s0 + lq[b]])) == 0
        elif causal and lq[b] > lk[b]:
            assert torch.count_nonzero(torch.from_numpy(got[s0:s0 + lq[b] - lk[b]])) == 0


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 100)])
def test_varlen_bit_identical_to_dense(causal, window):
    lq, lk = LENGTHS["ragged"]
    x = make_varlen_inputs("varlen_chunks_b5", seed=22, lengths_q=lq, lengths_k=lk)
    print(f"varlen == dense causal={causal} window={window}", flush=True)
    got = run_varlen(x, causal=causal, window=window)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    cq, ck = x["cu_q"], x["cu_k"]
    for b in range(len(lq)):
        if lq[b] == 0 or lk[b] == 0 or (causal and lk[b] < lq[b]):
            continue  # the dense entry point needs L, S >= 1 and a non-negative causal offset
        qd = q[cq[b]:cq[b + 1]].permute(1, 0, 2).contiguous()[None]
        kd = k[ck[b]:ck[b + 1]].permute(1, 0, 2).contiguous()[None]
        vd = v[ck[b]:ck[b + 1]].permute(1, 0, 2).contiguous()[None]
        dense = pfa.prefill_attn_gqa(qd, kd, vd, scale=float(x["scale"]), causal=causal,
                                     causal_offset=(lk[b] - lq[b]) if causal else None, window=window)
        torch.cuda.synchronize()
        mine = got[cq[b]:cq[b + 1]].permute(1, 0, 2)[None]
        assert torch.equal(mine.view(torch.int16), dense.view(torch.int16)), f"sequence {b}"


def test_varlen_malformed_prefix_sums_stay_in_bounds():
    # bounds past total_q / total_k and a decreasing pair: the kernel clamps every bound into the
    # packed extents, so nothing outside O is written (values inside are unspecified)
    lq, lk = [40, 30, 20], [50, 30, 20]
    x = make_varlen_inputs("varlen_chunks_b5", seed=23, lengths_q=lq, lengths_k=lk)
    tq = x["total_q"]
    guard = torch.full((tq + 300, x["Hq"], x["D"]), 7.0, dtype=torch.bfloat16, device=DEV)
    out = guard[:tq]
    print("varlen malformed prefix sums", flush=True)
    run_varlen(x, out=out, cu_q=[0, 60, 10, tq + 200], cu_k=[0, 10**6, 5, x["total_k"] + 9], max_q=300)
    assert torch.all(guard[tq:] == 7.0)


def test_varlen_full_size_full_oracle():
    # the packed batched-prompt workload at full size, in the launch configuration the bench times;
    # every output element against the oracle
    x = make_varlen_inputs("varlen_causal_b8", seed=0)
    print(f"varlen full size total_q={x['total_q']}", flush=True)
    got = run_varlen(x).double().cpu().numpy()
    ref = oracle_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], x["scale"], True, 0,
                        workers=max(1, min(16, host_workers())))
    check_close(got, ref, "varlen_causal_b8")


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 100)])
def test_varlen_options_parity_and_skip_identity(D, causal, window):
    """Soft-cap and attention sinks on the packed layout against the oracle; skip == no-skip bit for
    bit; each sequence bit-identical to the dense entry point with the same options."""
    lq, lk = LENGTHS["ragged"]
    x = make_varlen_inputs("varlen_chunks_b5", seed=23, lengths_q=lq, lengths_k=lk, D=D)
    Hq = x["Hq"]
    sinks = (np.random.default_rng(24).standard_normal(Hq) * 2.0).astype(np.float32)
    sinks[0] = -np.inf
    print(f"varlen options D={D} causal={causal} window={window}", flush=True)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    cq, ck = dev_i32(x["cu_q"]), dev_i32(x["cu_k"])
    st = torch.from_numpy(sinks).to(DEV)
    kw = dict(scale=float(x["scale"]), causal=causal, window=window, softcap=4.0, sinks=st)
    got = pfa.prefill_attn_gqa_varlen(q, k, v, cq, ck, x["max_seqlen_q"], **kw)
    got_ns = pfa.prefill_attn_gqa_varlen(q, k, v, cq, ck, x["max_seqlen_q"], no_skip=True, **kw)
    torch.cuda.synchronize()
    ref = oracle_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], x["scale"], causal, window, softcap=4.0,
                        sinks=sinks.astype(np.float64))
    check_close(got.double().cpu().numpy(), ref, f"options D={D} causal={causal} W={window}")
    assert torch.equal(got.view(torch.int16), got_ns.view(torch.int16))
    c_q, c_k = x["cu_q"], x["cu_k"]
    for b in range(len(lq)):
        if lq[b] == 0 or lk[b] == 0 or (causal and lk[b] < lq[b]):
            continue
        qd = q[c_q[b]:c_q[b + 1]].permute(1, 0, 2).contiguous()[None]
        kd = k[c_k[b]:c_k[b + 1]].permute(1, 0, 2).contiguous()[None]
        vd = v[c_k[b]:c_k[b + 1]].permute(1, 0, 2).contiguous()[None]
        dense = pfa.prefill_attn_gqa(qd, kd, vd, scale=float(x["scale"]), causal=causal,
                                     causal_offset=(lk[b] - lq[b]) if causal else None, window=window,
                                     softcap=4.0, sinks=st)
        torch.cuda.synchronize()
        mine = got[c_q[b]:c_q[b + 1]].permute(1, 0, 2)[None]
        assert torch.equal(mine.view(torch.int16), dense.view(torch.int16)), f"sequence {b}"
