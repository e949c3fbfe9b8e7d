"""Build the gfx950 library in-tree: bit_expert_dequant_amd/libmoe_dequant.so."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe_dequant.so")

SOURCES = ["moe_api.cpp", "moe_decode.hip", "moe_grouped.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *HIP_FLAGS, "-shared", f"-I{INCLUDE}", f"-I{CSRC}", *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        sys.stderr.write("\n".join(errs) + "\n")
        raise RuntimeError(f"hipcc failed with code {r.returncode}")
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
