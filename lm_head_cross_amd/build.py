"""Build the HIP shared libraries in-tree for gfx950 with hipcc: liborpo_head.so (the head) and
libmfma_peak.so (a measurement aid for bench.py --mfma-peak; the head never loads it)."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liborpo_head.so")
SOURCES = [os.path.join(HERE, "csrc", "orpo_head.hip")]
PEAK_LIB = os.path.join(HERE, "libmfma_peak.so")
PEAK_SOURCES = [os.path.join(HERE, "csrc", "mfma_peak.hip")]
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Keep the compiler from forming packed fp32 ops (v_pk_*_f32) in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(sources, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, *FLAGS, *sources, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    _compile(SOURCES, LIB, verbose)
    _compile(PEAK_SOURCES, PEAK_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
