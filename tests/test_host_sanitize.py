"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU, no GPU).

Builds the library source together with tests/host_abi_check.cpp into one executable, with the
sanitizers on the host pass only (device code is compiled as usual and never launched), and runs
the sweep: extreme sizes, every format pair, NaN / infinite scalars, unknown flags and the tiling
knob at its bounds. The sweep itself checks that workspace sizes and entry-point refusals agree;
the sanitizers check the size arithmetic for overflow and the host code for bad memory accesses.
"""
import os
import shutil
import subprocess

import pytest

from lm_head_cross_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.slow
def test_abi_argument_checks_under_host_sanitizers(tmp_path):
    if not os.path.exists(B.HIPCC) and not shutil.which(B.HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "host_abi_check")
    cmd = [B.HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-O1", "-Xarch_host", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(B.ROOT, "include"),
           *B.SOURCES, os.path.join(HERE, "host_abi_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, "build failed:\n" + r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "ok:" in r.stdout and ", 0 failures" in r.stdout, r.stdout
