"""Register budget of the head's kernels, read from the compiler's resource report (a gfx950
device-only compile of the library, no GPU needed).

The GEMM kernels run 512-thread workgroups (two waves per SIMD) and hold their accumulators in
registers across the K loop: a kernel that falls to one wave per SIMD, uses scratch (spilled
VGPRs), or spills many scalar registers to VGPR lanes is a performance regression even when its
results stay right. The scalar bounds sit far below what the epilogues once spilled when their
vocabulary-tail tests became 64 shared lane masks (212-354 scalars per forward kernel, 108-134 per
backward kernel) and above what they spill now.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "lm_head_cross_amd", "csrc", "orpo_head.hip")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def resources(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("res") / "dev.o"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-c", SRC, "-o", str(out),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    table, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            table[cur] = {}
            continue
        m = re.search(r"remark: \s*([A-Za-z ]+?)(?: \[[^\]]*\])?: (\w+) \[-Rpass", line)
        if m and cur:
            table[cur][m.group(1).strip()] = m.group(2)
    assert table, "no resource report parsed"
    return table


def _kernels(table, prefix):
    ks = {k: v for k, v in table.items() if k.startswith(prefix)}
    assert ks, prefix
    return ks


def test_no_kernel_uses_scratch_or_spills_vgprs(resources):
    for name, res in resources.items():
        if not name.startswith("_ZN4orpo"):
            continue
        assert res.get("ScratchSize") == "0", (name, res)
        assert res.get("VGPRs Spill") == "0", (name, res)


def test_gemm_kernels_keep_two_waves_per_simd(resources):
    for prefix in ("_ZN4orpo10fwd_kernel", "_ZN4orpo10bwd_kernel"):
        for name, res in _kernels(resources, prefix).items():
            assert int(res["Occupancy"]) >= 2, (name, res)


def test_scalar_spills_stay_small(resources):
    # Forward: up to 40. The running-maximum variants with per-tile maxima park the 16 LDS
    # addresses of their direct loads in VGPR lanes (one v_readlane per load, the cost of the
    # v_readfirstlane each load took when the addresses were computed per lane).
    for name, res in _kernels(resources, "_ZN4orpo10fwd_kernel").items():
        assert int(res["SGPRs Spill"]) <= 40, (name, res["SGPRs Spill"])
    for name, res in _kernels(resources, "_ZN4orpo10bwd_kernel").items():
        # The last template flag selects FP8 logit operands (more live scale state).
        f8 = name.endswith("ELb1EEEvNS_7BwdArgsE")
        assert int(res["SGPRs Spill"]) <= (64 if f8 else 8), (name, res["SGPRs Spill"])
