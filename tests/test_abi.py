"""C-ABI tests that need no GPU: the library loads, exports what include/pfa.h declares, and every
invalid argument is rejected on the host with its status code before anything is launched."""
import ctypes
import math
import os
import re

import pytest

import prefill_attention_amd as pfa
from prefill_attention_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pfa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pfa.LIB_PATH):
        from prefill_attention_amd.build import build_library
        build_library()
    return pfa.library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def header_defines():
    text = open(HEADER).read()
    vals = dict(re.findall(r"#define\s+(PFA_\w+)\s+\(?(-?\d+)u?\)?", text))
    enum = dict(re.findall(r"(PFA_(?:OK|ERR_\w+))\s*=\s*(\d+)", text))
    return {k: int(v) for k, v in vals.items()}, {k: int(v) for k, v in enum.items()}


def test_exports_every_declared_symbol(lib):
    funcs = header_functions()
    assert set(funcs) == set(pfa.EXPORTS), funcs
    for name in funcs:
        assert hasattr(lib, name), name


def test_binding_constants_match_header(lib):
    defines, enum = header_defines()
    assert defines["PFA_NO_CAUSAL"] == pfa.NO_CAUSAL
    assert defines["PFA_FLAG_NO_SKIP"] == pfa.FLAG_NO_SKIP
    assert defines["PFA_MAX_LEN"] == pfa.MAX_LEN
    assert defines["PFA_VERSION"] == pfa.version()
    assert {v: k for k, v in enum.items()} == pfa.STATUS


def test_status_strings(lib):
    for code in list(pfa.STATUS) + [99, -1]:
        s = pfa.status_str(code)
        assert isinstance(s, str) and s
    assert pfa.status_str(0) == "ok"
    assert pfa.status_str(99) == "unknown status"


# Fake, 16-byte aligned, non-overlapping "device" addresses: validation never dereferences them and
# returns before any HIP call when an argument is invalid.
A = 1 << 40
Q, K, V, O, M = A, 2 * A, 3 * A, 4 * A, 5 * A
GOOD = dict(q=Q, k=K, v=V, B=1, Hq=4, Hkv=2, L=33, S=47, D=128, scale=0.088, off=14, window=0,
            mask=None, o=O, stream=None, flags=0)


def call(**kw):
    a = dict(GOOD)
    a.update(kw)
    return pfa.prefill_attn_gqa_raw(a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["L"], a["S"],
                                    a["D"], a["scale"], a["off"], a["window"], a["mask"], a["o"],
                                    a["stream"], a["flags"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(o=0), 1),
    (dict(B=0), 2), (dict(Hq=0), 2), (dict(Hkv=-1), 2), (dict(L=0), 2), (dict(S=0), 2), (dict(D=0), 2),
    (dict(B=2 ** 31 - 1, Hq=2 ** 31 - 1, L=2 ** 31 - 1, Hkv=1), 2),
    (dict(S=2 ** 30 + 1), 2), (dict(L=2 ** 30 + 1), 2), (dict(S=2 ** 31 - 1), 2),
    (dict(Hq=6, Hkv=4), 3), (dict(Hq=7, Hkv=2), 3),
    (dict(D=96), 4), (dict(D=256), 4), (dict(D=32), 4),
    (dict(off=-1, window=5), 5),
    (dict(scale=float("nan")), 10), (dict(scale=float("inf")), 10), (dict(scale=0.0), 10), (dict(scale=-0.1), 10),
    (dict(q=Q + 8), 6), (dict(k=K + 2), 6), (dict(v=V + 4), 6), (dict(o=O + 1), 6),
    (dict(o=Q), 7), (dict(o=Q + 16), 7), (dict(o=K + 4096), 7), (dict(o=V - 16), 7), (dict(mask=O + 3), 7),
    (dict(flags=2), 9), (dict(flags=0x80000000), 9),
], ids=lambda x: str(x))
def test_invalid_arguments_rejected(lib, kw, code):
    assert call(**kw) == code


def test_validation_order(lib):
    # null beats size beats gqa beats head dim beats mask args beats scale beats align beats alias
    assert call(q=0, B=0) == 1
    assert call(B=0, Hq=7) == 2
    assert call(Hq=7, D=96) == 3
    assert call(D=96, off=-1, window=3) == 4
    assert call(off=-1, window=3, scale=0.0) == 5
    assert call(scale=0.0, q=Q + 2) == 10
    assert call(q=Q + 2, o=K) == 6
    assert call(o=K, flags=4) == 7


def test_o_adjacent_to_inputs_is_not_alias(lib):
    # O may sit right after Q (half-open ranges); only a launch would follow, so check the rule on
    # the mask instead, whose range is B*S bytes: a mask ending exactly at O is fine up to the
    # launch, which needs a GPU, so assert only that the alias code is not returned.
    q_bytes = 1 * 4 * 33 * 128 * 2
    rc = call(q=O - q_bytes, k=K, v=V, o=O, flags=2)   # flags error proves alias check passed
    assert rc == 9


def test_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 4, 8, 128, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        pfa.prefill_attn_gqa(q, k, k)
    with pytest.raises(ValueError, match="bfloat16"):
        pfa.prefill_attn_gqa(q.float(), k, k)
    with pytest.raises(TypeError):
        pfa.prefill_attn_gqa([1], k, k)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(_binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _binding.library()


# ---- packed variable-length entry point ----
CQ, CK = 6 * A, 7 * A
VGOOD = dict(q=Q, k=K, v=V, cq=CQ, ck=CK, n=3, maxq=40, tq=100, tk=120, Hq=4, Hkv=2, D=128,
             scale=0.088, causal=1, window=0, o=O, stream=None)


def vcall(**kw):
    a = dict(VGOOD)
    a.update(kw)
    return pfa.prefill_attn_gqa_varlen_raw(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["n"], a["maxq"],
                                           a["tq"], a["tk"], a["Hq"], a["Hkv"], a["D"], a["scale"],
                                           a["causal"], a["window"], a["o"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(o=0), 1), (dict(cq=0), 1), (dict(ck=0), 1),
    (dict(n=0), 2), (dict(maxq=0), 2), (dict(tq=0), 2), (dict(tk=0), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2),
    (dict(D=0), 2), (dict(maxq=2 ** 30 + 1), 2), (dict(n=2 ** 31 - 1), 2),
    (dict(Hq=2 ** 18, Hkv=2 ** 18), 2),
    (dict(Hq=2 ** 17, Hkv=2 ** 17), 2),     # a 64-key tile of packed rows would span exactly 2^31 bytes
    (dict(maxq=2 ** 30, n=2 ** 20, Hq=64, Hkv=64), 2),
    (dict(Hq=6, Hkv=4), 3),
    (dict(D=96), 4),
    (dict(causal=0, window=8), 5),
    (dict(scale=float("nan")), 10), (dict(scale=0.0), 10),
    (dict(q=Q + 8), 6), (dict(o=O + 2), 6), (dict(cq=CQ + 2), 6), (dict(ck=CK + 1), 6),
    (dict(o=Q), 7), (dict(o=K + 16), 7), (dict(o=V), 7), (dict(cq=O + 4), 7), (dict(ck=O + 100 * 4 * 128 * 2 - 4), 7),
], ids=lambda x: str(x))
def test_varlen_invalid_arguments_rejected(lib, kw, code):
    assert vcall(**kw) == code


def test_varlen_prefix_sums_adjacent_to_o_are_not_alias(lib):
    # cu buffers may sit right after O ([O, O + total_q*Hq*D*2) is half-open). An unknown flag bit is
    # checked after the alias rule, so PFA_ERR_FLAGS proves the alias check passed, and the call is
    # stopped before anything could be launched at these fake addresses.
    o_bytes = 100 * 4 * 128 * 2
    a = dict(VGOOD, cq=O + o_bytes, ck=O + o_bytes + 16)
    rc = pfa.prefill_attn_gqa_varlen_raw(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["n"], a["maxq"], a["tq"],
                                         a["tk"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"], a["window"],
                                         a["o"], a["stream"], flags=2)
    assert rc == 9


def test_varlen_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(10, 4, 128, dtype=torch.bfloat16)
    k = torch.zeros(12, 2, 128, dtype=torch.bfloat16)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match="3-D bfloat16 GPU"):
        pfa.prefill_attn_gqa_varlen(q, k, k, cu, cu, 10)


# ---- short-query (decode) entry point ----
WS = 8 * A
DGOOD = dict(GOOD, L=4, S=1000, off=996, ws=WS, wsb=None)


def dcall(**kw):
    a = dict(DGOOD)
    a.update(kw)
    need = pfa.decode_workspace_bytes(a["B"], a["Hq"], a["Hkv"], a["L"], a["S"], a["D"])
    wsb = need if a["wsb"] is None else a["wsb"]
    return pfa.prefill_attn_gqa_decode_raw(a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["L"], a["S"],
                                           a["D"], a["scale"], a["off"], a["window"], a["mask"], a["o"], a["ws"],
                                           wsb, a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(o=0), 1), (dict(ws=0), 1),
    (dict(L=0), 2), (dict(S=0), 2), (dict(L=65), 2), (dict(B=2 ** 21), 2),
    (dict(Hq=6, Hkv=4), 3), (dict(D=96), 4), (dict(off=-1, window=5), 5), (dict(scale=0.0), 10),
    (dict(ws=WS + 8), 6), (dict(q=Q + 2), 6),
    (dict(wsb=0), 11), (dict(wsb=-1), 11),
    (dict(ws=Q), 7), (dict(ws=O - 16), 7), (dict(ws=K + 64), 7),
], ids=lambda x: str(x))
def test_decode_invalid_arguments_rejected(lib, kw, code):
    assert dcall(**kw) == code


def wscall(**kw):
    a = dict(GOOD)
    a.update(kw)
    need = pfa.prefill_workspace_bytes(a["B"], a["Hq"], a["Hkv"], a["L"], a["S"], a["D"])
    wsb = need if a.get("wsb") is None else a["wsb"]
    return pfa.prefill_attn_gqa_ws_raw(a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["L"], a["S"], a["D"],
                                       a["scale"], a["off"], a["window"], a["mask"], a["o"], a.get("ws", WS), wsb,
                                       a["stream"], a.get("flags", 0))


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(ws=0), 1), (dict(L=0), 2), (dict(Hq=6, Hkv=4), 3), (dict(D=96), 4),
    (dict(off=-1, window=5), 5), (dict(scale=0.0), 10), (dict(q=Q + 2), 6), (dict(ws=WS + 8), 6),
    (dict(wsb=0), 11), (dict(wsb=-1), 11),
    (dict(ws=Q), 7), (dict(ws=O - 16), 7), (dict(ws=K + 64), 7), (dict(o=Q), 7),
    (dict(flags=2), 9),
], ids=lambda x: str(x))
def test_prefill_ws_invalid_arguments_rejected(lib, kw, code):
    assert wscall(**kw) == code


def test_prefill_workspace_bytes_function(lib):
    # FP32 partial slots of the 256 split workgroups (two each) and one 4-byte counter per item
    # a 1 KiB counter region first, then the partial slots
    slots128 = 2 * 256 * 8 * 64 * (16 * 4 + 2) * 4
    assert pfa.prefill_workspace_bytes(1, 8, 1, 2048, 32768, 128) == 1024 + slots128
    assert pfa.prefill_workspace_bytes(1, 4, 2, 33, 47, 64) == 1024 + 2 * 256 * 8 * 64 * (16 * 2 + 2) * 4
    assert pfa.prefill_workspace_bytes(1, 48, 8, 1024, 4096, 128) == 1024 + slots128  # 192 blocks: split
    # more than 192 query blocks: one workgroup per block, no workspace used (a 16-byte token)
    assert pfa.prefill_workspace_bytes(1, 56, 8, 2048, 8192, 128) == 16
    assert pfa.prefill_workspace_bytes(1, 193, 1, 256, 4096, 64) == 16
    for bad in [(0, 32, 8, 100, 100, 128), (1, 30, 8, 100, 100, 128), (1, 32, 8, 100, 100, 96), (1, 32, 8, 0, 100, 128)]:
        assert pfa.prefill_workspace_bytes(*bad) == -1, bad


def nacall(**kw):
    a = dict(DGOOD)
    a.update(kw)
    opts = pfa.Options(a.get("flags", 0), a.get("softcap", 0.0), a.get("bias"), 0, 0, 0, None, None, 0, 0, 0, 0, 0)
    return pfa.library().prefill_attn_gqa_decode_noalloc(
        a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["L"], a["S"], a["D"], ctypes.c_float(a["scale"]),
        a["off"], a["window"], a["mask"], a["o"], None, ctypes.byref(opts))


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(o=0), 1), (dict(L=0), 2), (dict(L=65), 2), (dict(Hq=6, Hkv=4), 3),
    (dict(D=96), 4), (dict(scale=0.0), 10), (dict(q=Q + 2), 6), (dict(o=Q), 7), (dict(flags=1), 9),
    (dict(bias=8 * A), 5),
    # the shape needs more partials than the library's 64 MiB scratch array holds
    (dict(B=64, Hq=64, Hkv=8, L=16, S=131072, off=131056), 11),
], ids=lambda x: str(x))
def test_decode_noalloc_invalid_arguments_rejected(lib, kw, code):
    assert nacall(**kw) == code


def test_decode_noalloc_scratch_limit_matches_workspace_rule(lib):
    assert pfa.decode_workspace_bytes(64, 64, 8, 16, 131072, 128) > pfa.DECODE_SCRATCH_BYTES
    assert pfa.decode_workspace_bytes(8, 32, 8, 64, 32768, 128) <= pfa.DECODE_SCRATCH_BYTES


def test_decode_workspace_too_small_by_one_byte(lib):
    need = pfa.decode_workspace_bytes(1, 4, 2, 4, 1000, 128)
    assert need > 0 and need % 16 == 0
    assert dcall(wsb=need - 1) == 11


def test_decode_workspace_bytes_function(lib):
    defines, _ = header_defines()
    assert defines["PFA_DECODE_MAX_L"] == pfa.DECODE_MAX_L
    assert defines["PFA_DECODE_SCRATCH_BYTES"] == pfa.DECODE_SCRATCH_BYTES
    assert pfa.decode_workspace_bytes(1, 32, 8, 1, 32768, 128) > 0
    for bad in [(0, 32, 8, 1, 100, 128), (1, 32, 8, 0, 100, 128), (1, 32, 8, 65, 100, 128), (1, 30, 8, 1, 100, 128),
                (1, 32, 8, 1, 100, 96), (1, 32, 8, 1, 0, 128)]:
        assert pfa.decode_workspace_bytes(*bad) == -1, bad
    # a pure function of the shape, growing with the rows kept per partial
    assert pfa.decode_workspace_bytes(1, 32, 8, 4, 4096, 128) == pfa.decode_workspace_bytes(1, 32, 8, 4, 4096, 128)
    assert pfa.decode_workspace_bytes(1, 32, 8, 8, 4096, 128) > pfa.decode_workspace_bytes(1, 32, 8, 1, 4096, 128)


# ---- rotating-cache entry point ----
KN, VN, KR, VR = 9 * A, 10 * A, 11 * A, 12 * A
RGOOD = dict(q=Q, kn=KN, vn=VN, kr=KR, vr=VR, B=1, Hq=8, Hkv=2, L=16, pos0=5000, ring=1088, D=128,
             scale=0.088, window=1024, o=O, stream=None)


def rcall(**kw):
    a = dict(RGOOD)
    a.update(kw)
    return pfa.prefill_attn_gqa_ring_raw(a["q"], a["kn"], a["vn"], a["kr"], a["vr"], a["B"], a["Hq"], a["Hkv"],
                                         a["L"], a["pos0"], a["ring"], a["D"], a["scale"], a["window"], a["o"],
                                         a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(kn=0), 1), (dict(vr=0), 1), (dict(o=0), 1),
    (dict(L=0), 2), (dict(pos0=-1), 2), (dict(ring=0), 2), (dict(pos0=2 ** 30), 2),
    (dict(Hq=6, Hkv=4), 3), (dict(D=96), 4), (dict(scale=float("nan")), 10),
    (dict(ring=1038), 12),                      # < window - 1 + L = 1039
    (dict(ring=63, window=8, L=4), 12),         # < 64 slots
    (dict(window=0, ring=4096), 12),            # no window: needs pos0 + L = 5016 slots
    (dict(kr=KR + 2), 6), (dict(o=O + 8), 6),
    (dict(kr=Q), 7), (dict(vr=KN + 64), 7), (dict(o=KR), 7), (dict(kr=VR - 1024), 7),
], ids=lambda x: str(x))
def test_ring_invalid_arguments_rejected(lib, kw, code):
    assert rcall(**kw) == code


@pytest.mark.parametrize("D,ring,code", [
    (128, 2 ** 23, 2), (128, 2 ** 23 + 64, 2), (64, 2 ** 24, 2),   # one (b, KV head) ring >= 2 GiB
    (128, 2 ** 23 - 64, 7), (64, 2 ** 24 - 64, 7),                 # just under: the planted alias is next
])
def test_ring_byte_offsets_stay_in_31_bits(lib, D, ring, code):
    # ring slots are addressed with 32-bit byte offsets; a ring of 2^31 bytes or more is refused
    assert rcall(D=D, ring=ring, pos0=100, L=16, window=0, kr=4 * A, vr=7 * A, q=8 * A, kn=9 * A, vn=10 * A,
                 o=8 * A) == code


def test_ring_capacity_rule_counts_only_existing_keys(lib):
    # pos0 + L <= ring: every key fits even though window - 1 + L would not; the next error after the
    # capacity check is an alias planted on purpose
    assert rcall(pos0=100, L=16, window=4096, ring=128, o=Q) == 7
    assert rcall(pos0=200, L=16, window=4096, ring=128, o=Q) == 12


# ---- options (soft-capping) ----
@pytest.mark.parametrize("softcap,code", [(float("nan"), 10), (float("inf"), 10), (-1.0, 10)])
def test_softcap_rejected(lib, softcap, code):
    a = dict(GOOD)
    assert pfa.prefill_attn_gqa_raw(a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["L"], a["S"], a["D"],
                                    a["scale"], a["off"], a["window"], a["mask"], a["o"], a["stream"], 0,
                                    softcap) == code
    d = dict(DGOOD)
    need = pfa.decode_workspace_bytes(d["B"], d["Hq"], d["Hkv"], d["L"], d["S"], d["D"])
    assert pfa.prefill_attn_gqa_decode_raw(d["q"], d["k"], d["v"], d["B"], d["Hq"], d["Hkv"], d["L"], d["S"],
                                           d["D"], d["scale"], d["off"], d["window"], d["mask"], d["o"], d["ws"],
                                           need, d["stream"], softcap) == code


def test_options_flags_checked(lib):
    a = dict(GOOD)
    # an unknown flag through the options struct, and any flag on the decode path
    assert pfa.prefill_attn_gqa_raw(a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["L"], a["S"], a["D"],
                                    a["scale"], a["off"], a["window"], a["mask"], a["o"], a["stream"], 2, 5.0) == 9
    d = dict(DGOOD)
    need = pfa.decode_workspace_bytes(d["B"], d["Hq"], d["Hkv"], d["L"], d["S"], d["D"])
    assert pfa.prefill_attn_gqa_decode_raw(d["q"], d["k"], d["v"], d["B"], d["Hq"], d["Hkv"], d["L"], d["S"],
                                           d["D"], d["scale"], d["off"], d["window"], d["mask"], d["o"], d["ws"],
                                           need, d["stream"], 0.0, 1) == 9


def test_options_layout_matches_header(tmp_path):
    """The ctypes mirror of struct pfa_options has the header's size and field offsets (the header
    compiled by the host C compiler)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    fields = [f[0] for f in pfa.Options._fields_]
    src = tmp_path / "layout.c"
    body = "".join(f'  printf("%s %zu\\n", "{f}", offsetof(pfa_options, {f}));\n' for f in fields)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "pfa.h"\nint main(void) {\n'
                   '  printf("size %zu\\n", sizeof(pfa_options));\n' + body + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                      text=True).stdout.splitlines())
    assert int(out["size"]) == ctypes.sizeof(pfa.Options)
    for f in fields:
        assert int(out[f]) == getattr(pfa.Options, f).offset, f


BIAS = 13 * A


def bcall(bias=BIAS, strides=(0, 0, 48), **kw):
    a = dict(GOOD)
    a.update(kw)
    return pfa.prefill_attn_gqa_raw(a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["L"], a["S"], a["D"],
                                    a["scale"], a["off"], a["window"], a["mask"], a["o"], a["stream"], 0, 0.0,
                                    bias, strides)


@pytest.mark.parametrize("kw,code", [
    (dict(mask=M), 5),                                   # not with a key mask
    (dict(strides=(0, 0, -4)), 2), (dict(strides=(-4, 0, 48)), 2),
    (dict(strides=(0, 0, 2 ** 28)), 2),                 # one (b, h) block too large
    (dict(bias=BIAS + 4), 6), (dict(strides=(0, 0, 50)), 6), (dict(strides=(2, 0, 48)), 6),
    (dict(bias=O), 7), (dict(bias=O - 64), 7),
], ids=lambda x: str(x))
def test_bias_rejected(lib, kw, code):
    assert bcall(**kw) == code


def test_bias_not_on_decode(lib):
    d = dict(DGOOD)
    need = pfa.decode_workspace_bytes(d["B"], d["Hq"], d["Hkv"], d["L"], d["S"], d["D"])
    opts = pfa.Options(0, 0.0, BIAS, 0, 0, 1000)
    lib_ = pfa.library()
    rc = lib_.prefill_attn_gqa_decode_opt(d["q"], d["k"], d["v"], d["B"], d["Hq"], d["Hkv"], d["L"], d["S"], d["D"],
                                          ctypes.c_float(d["scale"]), d["off"], d["window"], None, d["o"], d["ws"],
                                          need, None, ctypes.byref(opts))
    assert rc == 5


SINKS = 14 * A
SEL = 15 * A


def ocall(sinks=None, sel=None, blocks=(64, 64), sel_strides=(0, 0, 1), **kw):
    a = dict(GOOD)
    a.update(kw)
    return pfa.prefill_attn_gqa_raw(a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["L"], a["S"], a["D"],
                                    a["scale"], a["off"], a["window"], a["mask"], a["o"], a["stream"], 0, 0.0,
                                    a.get("bias"), a.get("bias_strides", (0, 0, 48)), sinks, sel, blocks,
                                    sel_strides)


@pytest.mark.parametrize("kw,code", [
    (dict(sinks=SINKS + 2), 6),                          # sink logits: 4-byte aligned
    (dict(sinks=O + 8), 7), (dict(sinks=O - 8), 7),     # and not overlapping O
    (dict(sel=SEL, blocks=(16, 64)), 2), (dict(sel=SEL, blocks=(48, 64)), 2),   # block_q % 32
    (dict(sel=SEL, blocks=(32, 32)), 2), (dict(sel=SEL, blocks=(32, 96)), 2),   # block_k % 64
    (dict(sel=SEL, blocks=(0, 64)), 2), (dict(sel=SEL, sel_strides=(0, -1, 1)), 2),
    (dict(sel=SEL, sel_strides=(1 << 62, 0, 1), B=2), 2),
    (dict(sel=SEL, mask=M), 5), (dict(sel=SEL, bias=BIAS), 5),  # not with a key mask or a bias
    (dict(sel=O), 7), (dict(sel=O - 1, blocks=(32, 64)), 7),  # rows 0-31 and 32: 2 bytes from O - 1
], ids=lambda x: str(x))
def test_sinks_and_block_bitmap_rejected(lib, kw, code):
    assert ocall(**kw) == code


def test_block_bitmap_not_on_decode(lib):
    d = dict(DGOOD)
    need = pfa.decode_workspace_bytes(d["B"], d["Hq"], d["Hkv"], d["L"], d["S"], d["D"])
    opts = pfa.Options(0, 0.0, None, 0, 0, 0, None, SEL, 32, 64, 0, 0, 1)
    rc = pfa.library().prefill_attn_gqa_decode_opt(
        d["q"], d["k"], d["v"], d["B"], d["Hq"], d["Hkv"], d["L"], d["S"], d["D"], ctypes.c_float(d["scale"]),
        d["off"], d["window"], None, d["o"], d["ws"], need, None, ctypes.byref(opts))
    assert rc == 5
    assert pfa.prefill_attn_gqa_decode_raw(d["q"], d["k"], d["v"], d["B"], d["Hq"], d["Hkv"], d["L"], d["S"],
                                           d["D"], d["scale"], d["off"], d["window"], None, d["o"], d["ws"],
                                           need, None, 0.0, 0, O + 2) == 6


def vocall(flags=0, softcap=0.0, sinks=None, bias=None, sel=None):
    a = dict(VGOOD)
    opts = pfa.Options(flags, softcap, bias, 0, 0, 0, sinks, sel, 32 if sel else 0, 64 if sel else 0, 0, 0, 1)
    return pfa.library().prefill_attn_gqa_varlen_opt(
        a["q"], a["k"], a["v"], a["cq"], a["ck"], a["n"], a["maxq"], a["tq"], a["tk"], a["Hq"], a["Hkv"], a["D"],
        ctypes.c_float(a["scale"]), 1 if a["causal"] else 0, a["window"], a["o"], None, ctypes.byref(opts))


@pytest.mark.parametrize("kw,code", [
    (dict(flags=2), 9), (dict(softcap=-1.0), 10), (dict(softcap=float("inf")), 10),
    (dict(bias=BIAS), 5), (dict(sel=SEL), 5),            # per dense row: not on the packed layout
    (dict(sinks=SINKS + 2), 6), (dict(sinks=O + 4), 7),
], ids=lambda x: str(x))
def test_varlen_options_rejected(lib, kw, code):
    assert vocall(**kw) == code


def rocall(flags=0, softcap=0.0, sinks=None, bias=None, sel=None):
    a = dict(RGOOD)
    opts = pfa.Options(flags, softcap, bias, 0, 0, 0, sinks, sel, 32 if sel else 0, 64 if sel else 0, 0, 0, 1)
    return pfa.library().prefill_attn_gqa_ring_opt(
        a["q"], a["kn"], a["vn"], a["kr"], a["vr"], a["B"], a["Hq"], a["Hkv"], a["L"], a["pos0"], a["ring"], a["D"],
        ctypes.c_float(a["scale"]), a["window"], a["o"], None, ctypes.byref(opts))


@pytest.mark.parametrize("kw,code", [
    (dict(flags=2), 9), (dict(softcap=-1.0), 10), (dict(bias=BIAS), 5), (dict(sel=SEL), 5),
    (dict(sinks=SINKS + 2), 6), (dict(sinks=O + 4), 7),
    (dict(sinks=KR + 64), 7), (dict(sinks=VR), 7),        # the rings are written before the sinks are read
], ids=lambda x: str(x))
def test_ring_options_rejected(lib, kw, code):
    assert rocall(**kw) == code
