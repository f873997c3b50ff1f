"""The entry points allocate nothing, synchronise nothing and launch only their own kernels on the
caller's stream, so they can be captured into a HIP graph. Capture each one (outputs and workspace
allocated beforehand), replay the graph several times with eager work and synchronisations in
between, and check every replay bit for bit against the eager call."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import prefill_attention_amd as pfa  # noqa: E402
from workloads import make_inputs, make_varlen_inputs  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def replay_matches(fn, out, reps=3):
    fn()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    for r in range(reps):
        out.zero_()
        junk = torch.randn(1 << 16, device=DEV) * float(r)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        del junk


def test_graph_prefill_and_softcap():
    x = make_inputs(dict(B=1, Hq=8, Hkv=2, D=128, L=300, S=900, causal_offset=600, window=0, amp=1.0,
                         key_padding=None), seed=71)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    out = torch.empty_like(q)
    print("graph: prefill", flush=True)
    replay_matches(lambda: pfa.prefill_attn_gqa(q, k, v, causal_offset=600, out=out), out)
    replay_matches(lambda: pfa.prefill_attn_gqa(q, k, v, causal_offset=600, softcap=5.0, out=out), out)


def test_graph_varlen():
    x = make_varlen_inputs("varlen_chunks_b5", seed=72)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    cq = torch.from_numpy(x["cu_q"]).to(DEV)
    ck = torch.from_numpy(x["cu_k"]).to(DEV)
    out = torch.empty_like(q)
    print("graph: varlen", flush=True)
    replay_matches(lambda: pfa.prefill_attn_gqa_varlen(q, k, v, cq, ck, x["max_seqlen_q"], out=out), out)


def test_graph_decode():
    x = make_inputs(dict(B=1, Hq=32, Hkv=8, D=128, L=1, S=9000, causal_offset=8999, window=0, amp=1.0,
                         key_padding=None), seed=73)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    out = torch.empty_like(q)
    ws = torch.empty(pfa.decode_workspace_bytes(1, 32, 8, 1, 9000, 128), dtype=torch.uint8, device=DEV)
    print("graph: decode", flush=True)
    replay_matches(lambda: pfa.prefill_attn_gqa_decode(q, k, v, causal_offset=8999, out=out, workspace=ws), out)
