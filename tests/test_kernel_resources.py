"""Register and scratch budgets of the gfx950 kernels, from the compiler's own resource
report (no GPU needed: hipcc cross-compiles the device code here).

A kernel that spills, or that keeps a captured array in private memory, runs its inner
loop through scratch and slows down several times over without any error; the parity
tests cannot see it. So every kernel must use no scratch, and the kernels designed for
two waves per SIMD must still fit two."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_io_aware_46_amd import build as fabuild

SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_bwd_rk.hip", "fa_bwd_rk_drop.hip", "fa_fwd_fp8.hip"]


def _report(src):
    cmd = [fabuild.HIPCC, *[f for f in fabuild.CFLAGS if f != "-fPIC"],
           *fabuild.SOURCE_FLAGS.get(src, []), "-x", "hip",
           "--cuda-device-only", "-c", os.path.join(fabuild.CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy "
                      r"\[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).split()[0]] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def resources():
    if not os.path.exists(fabuild.HIPCC) and shutil.which(fabuild.HIPCC) is None:
        pytest.skip("hipcc not available")
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        out = {}
        for k in ex.map(_report, SOURCES):
            out.update(k)
    return out


def test_every_kernel_was_reported(resources):
    names = " ".join(resources)
    for kernel in ("fwd_kernel", "bwd_pre_kernel", "bwd_dkdv_kernel", "bwd_dkdv_rk_kernel",
                   "bwd_dq_kernel", "fwd_fp8_kernel", "vt_fp8_kernel"):
        assert kernel in names, kernel


def test_no_kernel_uses_scratch(resources):
    bad = {k: v["ScratchSize"] for k, v in resources.items() if v.get("ScratchSize", 0)}
    assert not bad, f"kernels with scratch (bytes per lane): {bad}"


def test_two_wave_kernels_keep_two_waves_per_simd(resources):
    # Eight-wave workgroups (the template's last argument 8, mangled "Li8EE") are laid out
    # for two waves per SIMD; the four-wave ones (d = 256, and the dK/dV kernel that keeps
    # K and V in registers) for one.
    eight = {k: v for k, v in resources.items() if "Li8EEEv" in k}
    assert eight
    low = {k: v["Occupancy"] for k, v in eight.items() if v.get("Occupancy", 0) < 2}
    assert not low, f"eight-wave kernels below two waves per SIMD: {low}"


def test_kernels_that_share_a_cu_keep_their_occupancy(resources):
    # On the 64-wide layout: the four-wave forward (block tables) runs four waves per SIMD,
    # like the eight-wave one; the four-wave dQ kernel and the one-wave-per-SIMD dK/dV
    # kernel fit two workgroups per CU.
    want = {r"fwd_kernel.*ELi64ELi64ELb0E.*Li4EEEv": 4,
            r"bwd_dq_kernel.*ELi64ELi128ELb0E.*Li4EEEv": 2,
            r"bwd_dkdv_rk_kernel.*ELi64ELb0E": 2}
    for pat, occ in want.items():
        found = {k: v.get("Occupancy", 0) for k, v in resources.items() if re.search(pat, k)}
        assert found, pat
        low = {k: o for k, o in found.items() if o < occ}
        assert not low, f"below {occ} waves per SIMD: {low}"
