"""GPU parity of the key-split prefill (prefill_attn_gqa_ws): a fixed grid of workgroups takes equal
shares of the (query block, key tile) space, blocks split between workgroups leave FP32 partials in
the caller's workspace, and the last part merges them (tiny-llm Week 2 Day 5, Task 1 merge
equations). The split is taken for calls with at most 192 query blocks; others run the per-item grid.
Checked against the fp64 CPU oracle on every output element (|O_gpu - O_ref| <= 2e-2 + 2e-2 |O_ref|,
rms(err)/rms(ref) <= 1e-2), skip == NO_SKIP bit for bit, run-to-run bit identity with one reused
workspace, per-query-block counters left zero, and bit identity with the per-item call (workspace
untouched) where the split is not taken.
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
WORKERS = max(1, min(16, host_workers()))


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
    return msg


def workspace_for(q_shape, k_shape):
    B, Hq, L, D = q_shape
    need = pfa.prefill_workspace_bytes(B, Hq, k_shape[1], L, k_shape[2], D)
    assert need > 0
    return torch.zeros(need, dtype=torch.uint8, device=DEV)


def counters_zero(ws, shape=None):
    """The per-query-block counters at the start of the workspace (1 KiB) are all zero."""
    return bool(torch.all(ws[:1024] == 0))


def run(x, ws, no_skip=False, softcap=0.0, sinks=None):
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    mask = torch.from_numpy(x["key_mask"]).to(DEV) if x.get("key_mask") is not None else None
    off = x["causal_offset"]
    st = None if sinks is None else torch.from_numpy(sinks).to(DEV)
    out = pfa.prefill_attn_gqa(q, k, v, scale=float(x["scale"]), causal=off >= 0,
                               causal_offset=off if off >= 0 else None, window=x["window"], key_mask=mask,
                               no_skip=no_skip, softcap=softcap, sinks=st, workspace=ws)
    torch.cuda.synchronize()
    return out


SPLIT_MAX_BLOCKS = 192


def n_blocks(c):
    return c["B"] * c["Hq"] * -(-c["L"] // 256)


@pytest.mark.parametrize("name", ["mid_ctx_8k", "long_ctx_32k", "bidir_padded_b8", "sliding_w1024_d64"])
def test_many_blocks_run_the_per_item_grid(name):
    """Above 192 query blocks the workspace call is the per-item call: bit-identical output, and
    the workspace (partials and counters) is left as it was."""
    x = make_inputs(name, seed=0)
    assert n_blocks(x) > SPLIT_MAX_BLOCKS
    ws = workspace_for(x["q"].shape, x["k"].shape)
    print(f"[split not taken] {name}", flush=True)
    a = run(x, ws)
    b = run(x, None)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not bool(torch.any(ws != 0)), "workspace untouched"


@pytest.mark.parametrize("opt", ["bias", "block_sel"])
def test_bias_or_bitmap_run_the_per_item_grid(opt):
    """The workspace call with an additive bias or a block bitmap is the per-item call, also for a
    shape within the split limit."""
    c = dict(B=1, Hq=8, Hkv=2, D=128, L=600, S=1500, causal_offset=900, window=0, amp=1.0, key_padding=None)
    if opt == "bias":
        c["bias"] = "LS"
    else:
        c["block_sel"] = dict(block_q=64, block_k=128, density=0.5)
    x = make_inputs(c, seed=11)
    assert n_blocks(x) <= SPLIT_MAX_BLOCKS
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    kw = dict(scale=float(x["scale"]), causal_offset=x["causal_offset"])
    if opt == "bias":
        kw["bias"] = torch.from_numpy(x["bias"]).to(DEV)
    else:
        kw.update(block_sel=torch.from_numpy(x["block_sel"]).to(DEV), block_q=x["block_q"], block_k=x["block_k"])
    ws = workspace_for(tuple(q.shape), tuple(k.shape))
    a = pfa.prefill_attn_gqa(q, k, v, workspace=ws, **kw)
    b = pfa.prefill_attn_gqa(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not bool(torch.any(ws != 0)), "workspace untouched"


# fewer query blocks than compute units, the shapes the split is for: 8 query heads on one KV head,
# a 2048-row chunk after 30720 cached keys (64 blocks); 8 heads on 2 KV heads, 512 rows after 65024
# keys at D = 64 (16 blocks, each cut into 16 parts)
FEW_BLOCKS = {
    "h8_kv1_32k": dict(B=1, Hq=8, Hkv=1, D=128, L=2048, S=32768, causal_offset=30720, window=0, amp=1.0,
                       key_padding=None),
    "h8_kv2_64k_d64": dict(B=1, Hq=8, Hkv=2, D=64, L=512, S=65536, causal_offset=65024, window=0, amp=1.0,
                           key_padding=None),
    # bidirectional with key padding (the key-mask kernel), 128 blocks
    "b2_h8_bidir_padded_8k": dict(B=2, Hq=8, Hkv=2, D=128, L=2048, S=8192, causal_offset=-1, window=0, amp=1.0,
                                  key_padding=(1024, 8192)),
    # the sliding-window chunk on 8 heads, 64 blocks
    "h8_sliding_w1024": dict(B=1, Hq=8, Hkv=2, D=128, L=2048, S=3071, causal_offset=1023, window=1024, amp=1.0,
                             key_padding=None),
}


@pytest.mark.parametrize("name", sorted(FEW_BLOCKS))
def test_split_few_blocks(name):
    x = make_inputs(FEW_BLOCKS[name], seed=5)
    assert n_blocks(x) <= SPLIT_MAX_BLOCKS
    ws = workspace_for(x["q"].shape, x["k"].shape)
    print(f"[split few blocks] {name}", flush=True)
    a = run(x, ws)
    assert counters_zero(ws, x["q"].shape)
    b = run(x, ws)
    n = run(x, ws, no_skip=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "run to run"
    assert torch.equal(a.view(torch.int16), n.view(torch.int16)), "skip == no-skip"
    got = a.double().cpu().numpy()
    del a, b, n
    ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], x["causal_offset"], x["window"], x["key_mask"],
                      workers=WORKERS)
    print(check_close(got, ref, name), flush=True)


def random_cases(n=32, seed=91):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2, 8]))
        G = int(rng.choice([1, 2, 4, 7]))
        B = int(rng.integers(1, 4))
        D = int(rng.choice([64, 128]))
        L = int(rng.integers(1, 1400))
        S = int(rng.integers(1, 3000))
        kind = i % 4
        if kind == 0:
            off, W = S - L if S >= L else int(rng.integers(0, S + 1)), 0
        elif kind == 1:
            off, W = int(rng.integers(0, S + 200)), int(rng.choice([1, 5, 64, 300]))   # windows, some past S
        elif kind == 2:
            off, W = -1, 0
        else:
            off, W = max(0, S - L), int(rng.integers(1, 2000))
        kp = (1, S) if (i % 3 == 0 and S > 1) else None
        c = dict(B=B, Hq=Hkv * G, Hkv=Hkv, D=D, L=L, S=S, causal_offset=off, window=W, amp=1.0, key_padding=kp)
        if i % 8 == 7:   # above the split limit: the workspace call runs the per-item grid
            c.update(B=3, Hq=56, Hkv=8, L=max(L, 1025))
        else:
            while n_blocks(c) > SPLIT_MAX_BLOCKS:
                c["B"] = max(1, c["B"] - 1) if c["B"] > 1 else 1
                if n_blocks(c) > SPLIT_MAX_BLOCKS and c["B"] == 1:
                    c["Hq"] = c["Hkv"]
        out.append(c)
    return out


def test_split_random_shapes_one_workspace():
    """Ragged shapes (tails on both axes, windows that start past the last key, key padding,
    bidirectional, D = 64 and 128, fewer key tiles than workgroups) with soft-cap and sinks on some,
    all through one workspace sized for the largest: oracle parity, skip == no-skip bitwise,
    counters zero after every call."""
    cases = random_cases()
    need = max(pfa.prefill_workspace_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["S"], c["D"]) for c in cases)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    for i, c in enumerate(cases):
        x = make_inputs(c, seed=100 + i)
        softcap = 30.0 if i % 5 == 1 else 0.0
        sinks = (np.random.default_rng(i).standard_normal(c["Hq"]) * 2).astype(np.float32) if i % 4 == 3 else None
        print(f"[split random] {i} {c} softcap={softcap} sinks={sinks is not None}", flush=True)
        a = run(x, ws, softcap=softcap, sinks=sinks)
        n = run(x, ws, no_skip=True, softcap=softcap, sinks=sinks)
        assert torch.equal(a.view(torch.int16), n.view(torch.int16)), f"case {i}: skip == no-skip"
        assert counters_zero(ws, x["q"].shape)
        ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], x["causal_offset"], x["window"], x["key_mask"],
                          workers=WORKERS, softcap=softcap, sinks=None if sinks is None else sinks.astype(np.float64))
        got = a.double().cpu().numpy()
        check_close(got, ref, f"case {i}")
        empty = ~np.any(np.abs(ref) > 0, axis=-1)
        assert np.all(got[empty] == 0.0), f"case {i}: rows without keys are zeros"


def test_split_close_to_per_item_grid():
    # another summation boundary, so not bitwise; both within the oracle tolerance of each other
    x = make_inputs(FEW_BLOCKS["h8_kv1_32k"], seed=3)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    ws = workspace_for(tuple(q.shape), tuple(k.shape))
    a = pfa.prefill_attn_gqa(q, k, v, scale=float(x["scale"]), causal_offset=x["causal_offset"], workspace=ws)
    b = pfa.prefill_attn_gqa(q, k, v, scale=float(x["scale"]), causal_offset=x["causal_offset"])
    torch.cuda.synchronize()
    check_close(a.double().cpu().numpy(), b.double().cpu().numpy(), "split vs per-item grid")


def test_workspace_reused_across_head_sizes():
    """One zero-filled workspace through calls of both head sizes: a D = 128 call whose parts fill
    the whole partial region, then a D = 64 call (its partial slots sit elsewhere), then D = 128
    again. The counters live at a fixed place, so each call still merges exactly its own parts: each
    result matches the per-item call within the tolerance, and the repeated call is bit-identical."""
    big = make_inputs(FEW_BLOCKS["h8_kv1_32k"], seed=21)
    small = make_inputs(FEW_BLOCKS["h8_kv2_64k_d64"], seed=22)
    need = max(pfa.prefill_workspace_bytes(x["B"], x["Hq"], x["Hkv"], x["L"], x["S"], x["D"]) for x in (big, small))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    print("[split] workspace reused across head sizes", flush=True)
    a1 = run(big, ws)
    s1 = run(small, ws)
    a2 = run(big, ws)
    assert counters_zero(ws)
    assert torch.equal(a1.view(torch.int16), a2.view(torch.int16))
    for got, x, what in ((s1, small, "D=64 after D=128"), (a2, big, "D=128 after D=64")):
        ref = run(x, None)
        check_close(got.double().cpu().numpy(), ref.double().cpu().numpy(), what)
