"""Build liboscar.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m decode_attention_write_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "oscar")
LIB = os.path.join(PKG, "liboscar.so")

ARCH = "gfx950"
COMMON = [
    "hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-I", INCLUDE, "-I", CSRC,
]
# per-source extra flags; the write path never fuses multiply-add in the quantizer
SOURCES = {
    "oscar_host.cpp": [],
    "calibrate.cpp": [],
    "write.hip": ["-ffp-contract=off"],
    "decode.hip": [],
    "scratch.hip": [],
    # keep MFMA accumulators in arch VGPRs (no AGPR copies around the running rescale)
    "decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")


SYNTH_SRC = os.path.join(ROOT, "synth", "csrc", "gen.hip")
SYNTH_LIB = os.path.join(ROOT, "synth", "libsynth_gen.so")


def build_synth(verbose: bool = False) -> str:
    """The GPU twin of the seeded input generator (input drawing only, not part of liboscar)."""
    tmp = SYNTH_LIB + ".tmp"
    _run(["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-ffp-contract=off",
          SYNTH_SRC, "-o", tmp], verbose)
    os.replace(tmp, SYNTH_LIB)
    return SYNTH_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run(COMMON + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_synth(verbose=True))
