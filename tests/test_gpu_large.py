"""Keys beyond 4 GiB per KV head: 64-bit addressing of K and V in the prefill (dense and packed
layouts, one workgroup per block and the key split) and decode kernels, checked through a property
that holds at any size.

With K = 0 every visible score is 0, so the softmax is uniform over the visible keys; with V = 1 for
keys at or past 2^24 and 0 before, every output element of row i is the fraction of its visible keys
that lie past 2^24. Key 2^24 starts at byte 4 GiB of the head's K and V (128 bf16 per row), so a
byte offset kept in 32 bits would wrap to the zero rows at the start and give 0 instead.

The sums stay exact in FP32 (counts of ones below 2^24 per lane), so the only error is the final
BF16 rounding of the ratio.
"""
import pytest
import torch

import prefill_attention_amd as pfa

pytestmark = pytest.mark.gpu

DEV = "cuda"
D = 128
EDGE = 1 << 24                  # first key whose rows start at byte 4 GiB of a head
S = EDGE + (1 << 22)            # 20,971,520 keys: K and V of one head are 5 GiB each


@pytest.fixture(scope="module")
def kv():
    k = torch.zeros(1, 1, S, D, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    v[:, :, EDGE:, :] = 1.0
    torch.cuda.synchronize()
    yield k, v
    del k, v
    torch.cuda.empty_cache()


def expected_rows(L):
    # row i (causal offset S - L) sees keys 0 .. S - L + i
    n = torch.arange(L, dtype=torch.float64) + (S - L + 1)
    return ((n - EDGE) / n).view(1, 1, L, 1).expand(1, 1, L, D)


def check(out, L):
    got = out.double().cpu()
    ref = expected_rows(L)
    err = (got - ref).abs().max().item()
    # BF16 rounding of a value near 0.2 is at most 2^-11 (relative 2^-9)
    assert err <= 2e-3, f"max error {err:.3e}, got row 0 {got[0, 0, 0, :4].tolist()} expected {ref[0, 0, 0, 0].item():.6f}"


def test_prefill_dense_keys_past_4gib(kv):
    k, v = kv
    L = 32
    q = torch.randn(1, 1, L, D, device=DEV).to(torch.bfloat16)
    out = pfa.prefill_attn_gqa(q, k, v)  # causal, offset S - L
    torch.cuda.synchronize()
    check(out, L)


def test_prefill_packed_keys_past_4gib(kv):
    k, v = kv
    L = 32
    q = torch.randn(L, 1, D, device=DEV).to(torch.bfloat16)
    cu_q = torch.tensor([0, L], dtype=torch.int32, device=DEV)
    cu_k = torch.tensor([0, S], dtype=torch.int32, device=DEV)
    # packed layout [total, H, D]: with one KV head the dense [1, 1, S, D] buffer is the same memory
    out = pfa.prefill_attn_gqa_varlen(q, k.view(S, 1, D), v.view(S, 1, D), cu_q, cu_k, L)
    torch.cuda.synchronize()
    check(out.view(L, 1, 1, D).permute(1, 2, 0, 3), L)


def test_decode_keys_past_4gib(kv):
    k, v = kv
    L = 8
    q = torch.randn(1, 1, L, D, device=DEV).to(torch.bfloat16)
    ws = torch.empty(pfa.decode_workspace_bytes(1, 1, 1, L, S, D), dtype=torch.uint8, device=DEV)
    out = pfa.prefill_attn_gqa_decode(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    check(out, L)


def test_prefill_key_split_keys_past_4gib(kv):
    # one query block of one head: the key split cuts its 327,680 key tiles into 256 parts, most of
    # them past byte 4 GiB, whose partial counts the last part merges
    k, v = kv
    L = 32
    q = torch.randn(1, 1, L, D, device=DEV).to(torch.bfloat16)
    ws = torch.zeros(pfa.prefill_workspace_bytes(1, 1, 1, L, S, D), dtype=torch.uint8, device=DEV)
    out = pfa.prefill_attn_gqa(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    check(out, L)
