"""Build the gfx950 library in-tree: bit_expert_dequant_amd/libmoe_dequant.so.

Each source is compiled to an object on its own (in parallel, into _build/, where host-side checks
can relink them), then the objects are linked."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe_dequant.so")
OBJ_DIR = os.path.join(HERE, "_build")

SOURCES = ["moe_api.cpp", "moe_batched8.hip", "moe_shared_gu.hip", "moe_shared_gux.hip", "moe_shared_dn.hip", "moe_decode.hip", "moe_grouped.hip", "moe_layer.hip", "moe_quant.hip", "moe_tier.hip", "moe_cache.hip", "moe_static.hip", "moe_fused.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l]
    return r.returncode, errs


def build(verbose: bool = False) -> str:
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.basename(s) + ".o") for s in srcs]
    cmds = [["hipcc", *HIP_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, errs), s in zip(results, srcs):
        if rc != 0:
            sys.stderr.write("\n".join(errs) + "\n")
            raise RuntimeError(f"hipcc failed on {os.path.basename(s)} with code {rc}")
        if verbose and errs:
            sys.stderr.write("\n".join(errs) + "\n")
    tmp = LIB + ".tmp"
    link = ["hipcc", "--offload-arch=gfx950", "-shared", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link))
    rc, errs = _run(link)
    if rc != 0:
        sys.stderr.write("\n".join(errs) + "\n")
        raise RuntimeError(f"link failed with code {rc}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
