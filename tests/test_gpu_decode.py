"""GPU parity of the short-query (decode) entry point against the fp64 CPU oracle: the same
operation as prefill_attn_gqa (masks, head map, empty rows), computed with the key range split over
the chip and a fixed-order merge of the partials (tiny-llm Week 2 Day 5, Task 1 merge equations).

Tolerance as in test_gpu_parity.py: |O_gpu - O_ref| <= 2e-2 + 2e-2 |O_ref| elementwise and
rms(err)/rms(ref) <= 1e-2.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import prefill_attention_amd as pfa  # noqa: E402
from oracle import NO_CAUSAL, oracle_sdpa  # noqa: E402
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


def decode(x, workspace=None):
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    mask = torch.from_numpy(x["key_mask"]).to(DEV) if x.get("key_mask") is not None else None
    off = x["causal_offset"]
    out = pfa.prefill_attn_gqa_decode(q, k, v, scale=float(x["scale"]), causal=off >= 0,
                                      causal_offset=off if off >= 0 else None, window=x["window"], key_mask=mask,
                                      workspace=workspace)
    torch.cuda.synchronize()
    return out


# (name, B, Hq, Hkv, D, L, S, causal_offset, window, key padding)
CASES = [
    ("l1_s32k", 1, 32, 8, 128, 1, 32768, 32767, 0, None),
    ("l8_g7_s8k", 1, 56, 8, 128, 8, 8192, 8184, 0, None),    # 56 rows per KV head: two MFMA blocks
    ("l4_d64_window", 1, 32, 8, 64, 4, 3071, 3067, 1024, None),
    ("l2_bidir_keymask", 3, 8, 2, 128, 2, 5000, NO_CAUSAL, 0, (1, 5000)),
    ("l16_g8_rowgroups", 1, 16, 2, 128, 16, 700, 684, 0, None),  # 128 rows per KV head: two row groups
    ("l3_s33_offset0", 1, 4, 2, 128, 3, 33, 0, 0, None),
    ("l8_more_rows_than_keys", 1, 4, 4, 128, 8, 5, 0, 0, None),
    ("l1_s1", 2, 2, 1, 64, 1, 1, 0, 0, None),
    ("l64_window_d64", 1, 8, 8, 64, 64, 2000, 1936, 100, None),
    # exactly 32 rows per KV head (the register-K kernel's limit), a window and a ragged last tile
    ("l8_g4_rows32_window", 2, 16, 4, 128, 8, 1000, 992, 300, None),
    # one tile per split and keys shorter than a tile for some rows (padding steps of the split kernel)
    ("l2_g2_s70", 3, 4, 2, 128, 2, 70, 68, 0, None),
    # one visible key per row (window 1): the output is that key's value row, bit for bit
    ("l4_window1", 2, 8, 2, 128, 4, 300, 296, 1, None),
    ("l40_window1_rows160", 1, 16, 4, 64, 40, 1000, 960, 1, None),
    # rows whose window starts after their split's last key while a padding step of the
    # register-K kernel covers key S + 32 (a sentinel past S once made that key visible)
    ("l8_window1_s388_padding", 1, 8, 8, 128, 8, 388, 380, 1, None),
    ("l8_window3_s420", 1, 8, 8, 128, 8, 420, 412, 3, None),
]


def small_window_cases(n=24, seed=77):
    """Seeded random decode shapes with short windows (ragged key counts, 1 <= window < 64)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4]))
        D = int(rng.choice([64, 128]))
        L = int(rng.integers(1, 9))
        S = int(rng.integers(L, 1500))
        W = int(rng.integers(1, 64))
        out.append((f"win{i}", 1, Hkv * G, Hkv, D, L, S, S - L, W, None))
    return out


CASES += small_window_cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(case):
    name, B, Hq, Hkv, D, L, S, off, W, kp = case
    x = make_inputs(dict(B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, S=S, causal_offset=off, window=W, amp=1.0,
                         key_padding=kp), seed=31)
    print(f"decode parity {name}", flush=True)
    got = decode(x).double().cpu().numpy()
    ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], off, W, x["key_mask"], workers=16)
    check_close(got, ref, name)
    # rows that see no key are exact zeros
    empty = ~np.any(np.abs(ref) > 0, axis=-1)
    assert np.all(got[empty] == 0.0)
    if W == 1:  # row i sees only key i + off: P = 1, l = 1, and O is that value row exactly
        G = Hq // Hkv
        vbits = x["v"]
        for h in range(Hq):
            want = vbits[:, h // G, off:off + L, :]
            gotbits = torch.from_numpy(got[:, h].astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
            assert np.array_equal(gotbits.view(np.uint16), want.view(np.uint16)), f"{name}: head {h}"


def test_decode_deterministic_and_workspace_reuse():
    x = make_inputs(dict(B=1, Hq=32, Hkv=8, D=128, L=4, S=9000, causal_offset=8996, window=0, amp=1.0,
                         key_padding=None), seed=32)
    y = make_inputs(dict(B=2, Hq=8, Hkv=2, D=64, L=1, S=300, causal_offset=299, window=0, amp=1.0,
                         key_padding=None), seed=33)
    need = max(pfa.decode_workspace_bytes(1, 32, 8, 4, 9000, 128), pfa.decode_workspace_bytes(2, 8, 2, 1, 300, 64))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    print("decode determinism / workspace reuse", flush=True)
    a1 = decode(x, ws)
    b1 = decode(y, ws)
    a2 = decode(x, ws)
    assert torch.equal(a1.view(torch.int16), a2.view(torch.int16))
    check_close(b1.double().cpu().numpy(), oracle_sdpa(y["q"], y["k"], y["v"], y["scale"], 299, 0, None), "reuse")


def test_decode_matches_prefill_entry_point():
    x = make_inputs(dict(B=1, Hq=32, Hkv=8, D=128, L=8, S=4096, causal_offset=4088, window=0, amp=1.0,
                         key_padding=None), seed=34)
    print("decode vs prefill entry point", flush=True)
    d = decode(x).double().cpu().numpy()
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    p = pfa.prefill_attn_gqa(q, k, v, scale=float(x["scale"]), causal_offset=4088)
    torch.cuda.synchronize()
    check_close(d, p.double().cpu().numpy(), "decode vs prefill")


def test_decode_small_workspace_raises():
    x = make_inputs(dict(B=1, Hq=4, Hkv=2, D=128, L=1, S=100, causal_offset=99, window=0, amp=1.0,
                         key_padding=None), seed=35)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(pfa.PfaError, match="WORKSPACE"):
        decode(x, ws)
