"""GPU parity of the block bitmap (TensorFold PR, "What changes": MiniMax-M3's prompt attention adds
a block bitmap, SEL; read here as: key j is visible to row i of (b, h) only where
sel[b, h, i // block_q, j // block_k] is nonzero) on the prefill entry point, against the fp64
CPU oracle. Unselected key blocks are skipped whole; skip == no-skip bit for bit; an all-ones
bitmap gives the plain call's bits.

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


# (name, B, Hq, Hkv, D, L, S, causal_offset, window, block_q, block_k, density, bitmap shape, softcap, sinks)
CASES = [
    ("causal_bq32_bk64", 1, 8, 2, 128, 300, 900, 600, 0, 32, 64, 0.5, "BH", 0.0, False),
    ("bidir_bq256_bk128", 2, 4, 2, 128, 520, 700, -1, 0, 256, 128, 0.4, "B1", 0.0, False),
    ("window_d64_bq64_bk192", 1, 8, 4, 64, 400, 1000, 600, 200, 64, 192, 0.6, "1H", 0.0, False),
    ("softcap_bq128_bk64", 1, 4, 2, 128, 257, 700, 443, 0, 128, 64, 0.5, "Q", 4.0, False),
    ("sinks_bq96_bk320", 1, 8, 2, 128, 500, 1500, 1000, 0, 96, 320, 0.3, "BH", 0.0, True),
    ("sparse_rows_bq32_bk64", 1, 4, 4, 128, 200, 333, 133, 0, 32, 64, 0.1, "BH", 0.0, False),
]


def make_sel(rng, kind, B, Hq, nqb, nkb, density):
    shape = {"BH": (B, Hq, nqb, nkb), "B1": (B, 1, nqb, nkb), "1H": (1, Hq, nqb, nkb), "Q": (nqb, nkb)}[kind]
    return (rng.random(shape) < density).astype(np.uint8)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_bitmap_parity_and_skip_identity(case):
    name, B, Hq, Hkv, D, L, S, off, W, bq, bk, dens, kind, cap, with_sinks = case
    x = make_inputs(dict(B=B, Hq=Hq, Hkv=Hkv, D=D, L=L, S=S, causal_offset=off, window=W, amp=1.0,
                         key_padding=None), seed=91)
    rng = np.random.default_rng(92)
    nqb, nkb = -(-L // bq), -(-S // bk)
    sel = make_sel(rng, kind, B, Hq, nqb, nkb, dens)
    sinks = (rng.standard_normal(Hq) * 2.0).astype(np.float32) if with_sinks else None
    print(f"block bitmap {name}", flush=True)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    kw = dict(scale=float(x["scale"]), causal=off >= 0, causal_offset=off if off >= 0 else None, window=W,
              softcap=cap, sinks=None if sinks is None else torch.from_numpy(sinks).to(DEV))
    st = torch.from_numpy(sel).to(DEV)
    out = pfa.prefill_attn_gqa(q, k, v, block_sel=st, block_q=bq, block_k=bk, **kw)
    out_ns = pfa.prefill_attn_gqa(q, k, v, block_sel=st, block_q=bq, block_k=bk, no_skip=True, **kw)
    torch.cuda.synchronize()
    ref = oracle_sdpa(x["q"], x["k"], x["v"], x["scale"], off, W, None, workers=16, softcap=cap,
                      sinks=None if sinks is None else sinks.astype(np.float64), block_sel=sel, block_q=bq,
                      block_k=bk)
    got = out.double().cpu().numpy()
    check_close(got, ref, name)
    assert torch.equal(out.view(torch.int16), out_ns.view(torch.int16))
    empty = ~np.any(np.abs(ref) > 0, axis=-1)
    assert np.all(got[empty] == 0.0)


@pytest.mark.parametrize("bq,bk", [(32, 64), (256, 256)])
def test_all_ones_bitmap_is_plain(bq, bk):
    x = make_inputs(dict(B=1, Hq=8, Hkv=2, D=128, L=600, S=1300, causal_offset=700, window=0, amp=1.0,
                         key_padding=None), seed=93)
    q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    ones = torch.ones(-(-600 // bq), -(-1300 // bk), dtype=torch.uint8, device=DEV)
    print(f"block bitmap all ones {bq}x{bk}", flush=True)
    out = pfa.prefill_attn_gqa(q, k, v, causal_offset=700, block_sel=ones, block_q=bq, block_k=bk)
    plain = pfa.prefill_attn_gqa(q, k, v, causal_offset=700)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
