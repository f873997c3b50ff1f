"""Register budget of every GPU kernel, from the compiler's resource-usage remarks (CPU only: hipcc
cross-compiles the device code for gfx950 with the library's own flags).

A kernel that spills vector registers to scratch runs several times slower without any test of its
results noticing (a block-bitmap instantiation once spilled 269 VGPRs and ran 6.4 x slower). Every
prefill instantiation must keep all its vector registers; the decode path's register-K kernel at
D = 128 holds 256 VGPRs with a few spilled around its loop by design, and may not spill more.
"""
import os
import re
import subprocess

import pytest

from prefill_attention_amd import build

# kernel name prefix -> VGPRs it may spill (mangled names contain the template arguments)
ALLOWED_VGPR_SPILLS = {
    "_ZN12_GLOBAL__N_122pfa_decode_kreg_kernelILi128E": 7,
}


def kernel_resources(source: str) -> dict:
    """{mangled kernel name: (VGPRs spilled, SGPRs spilled)} of one source file."""
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [build.hipcc(), *flags, "--cuda-device-only", "-c", "-Rpass-analysis=kernel-resource-usage",
           os.path.join(build.CSRC, source), "-o", os.devnull]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    out, name = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = [0, 0]
            continue
        m = re.search(r"(VGPRs|SGPRs) Spill: (\d+)", line)
        if m and name is not None:
            out[name][0 if m.group(1) == "VGPRs" else 1] = int(m.group(2))
    return {k: tuple(v) for k, v in out.items()}


@pytest.mark.parametrize("source", ["pfa_kernel.hip", "pfa_decode.hip"])
def test_no_unexpected_vgpr_spills(source):
    res = kernel_resources(source)
    assert res, "no kernels found in the compiler remarks"
    if source == "pfa_kernel.hip":
        # every instantiation: 2 head sizes x 10 per-item modes + 2 x 4 split modes, and the ring append
        assert sum(1 for k in res if "pfa_prefill_kernel" in k) == 28, sorted(res)
    bad = []
    for name, (vgpr, _sgpr) in res.items():
        limit = next((v for k, v in ALLOWED_VGPR_SPILLS.items() if name.startswith(k)), 0)
        if vgpr > limit:
            bad.append(f"{name}: {vgpr} VGPRs spilled (allowed {limit})")
    assert not bad, "\n".join(bad)


def test_split_merge_loads_are_batched():
    """The key split's merge issues each part's partial loads together: when register pressure
    around the merge made the compiler wait for every load before issuing the next, a 16-part merge
    took 275 instead of 21 us (results unchanged, so only the code shows it)."""
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    res = subprocess.run([build.hipcc(), *flags, "--cuda-device-only", "-S", os.path.join(build.CSRC, "pfa_kernel.hip"),
                          "-o", "-"], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    funcs = re.split(r"\n(?=_ZN\S+:)", res.stdout)
    checked = 0
    for f in funcs:
        name = f.split(":", 1)[0]
        if "pfa_prefill_kernel" not in name or "Lb1E" not in name:
            continue
        lines = [l.strip() for l in f.splitlines()]
        loads = [i for i, l in enumerate(lines) if l.startswith("buffer_load_dword") and "sc1" in l]
        assert loads, f"{name}: no device-coherent partial loads found"
        waits = sum("vmcnt" in l for l in lines[loads[0]:loads[-1] + 1])
        assert waits <= 16, f"{name}: {waits} vmcnt waits among its {len(loads)} partial loads"
        checked += 1
    assert checked == 8, checked
