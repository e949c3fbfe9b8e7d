"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The library's host-only source (argument validation, the packer, workspace sizing, the expert-cache
  policy) is rebuilt with both sanitizers and linked with the HIP objects of the normal build; the host
  ABI tests then run against that copy in a process with the ASan runtime preloaded.
* The oracle's C is rebuilt with both sanitizers and its pins run against it.
A sanitizer report ends the child process with a failure status, which fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_expert_dequant_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ASAN_OPTIONS = "detect_leaks=0:verify_asan_link_order=0"
UBSAN_OPTIONS = "halt_on_error=1:print_stacktrace=1"
# host-side sanitizers only: on a hipcc line each sanitizer flag follows -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def run_child(code: str, env_extra: dict, timeout: int = 900) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env.update(env_extra)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def test_host_library_under_asan_and_ubsan(tmp_path):
    from bit_expert_dequant_amd import build as B
    hip_objs = [os.path.join(B.OBJ_DIR, os.path.basename(s) + ".o") for s in B.sources()
                if not s.endswith(".cpp")]
    if not all(os.path.exists(o) for o in hip_objs):
        B.build()
    api_o, lib = str(tmp_path / "api.o"), str(tmp_path / "libmoe_san.so")
    subprocess.run(["hipcc", "-O1", "-g", "-std=c++17", "-fPIC", *HOST_SAN, f"-I{INCLUDE}", f"-I{CSRC}", "-c",
                    os.path.join(CSRC, "moe_api.cpp"), "-o", api_o], check=True, capture_output=True)
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-shared-libasan", *HOST_SAN, api_o, *hip_objs,
                    "-o", lib], check=True, capture_output=True)
    runtime = subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                             check=True, capture_output=True, text=True).stdout.strip()
    assert os.path.exists(runtime), runtime
    code = ("import sys\nimport bit_expert_dequant_amd as M\n"
            f"M.LIB_PATH = {lib!r}\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_abi_host.py']))\n")
    r = run_child(code, {"LD_PRELOAD": runtime, "ASAN_OPTIONS": ASAN_OPTIONS, "UBSAN_OPTIONS": UBSAN_OPTIONS})
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert " passed" in r.stdout and "failed" not in r.stdout


def test_oracle_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", lib, "-lm"], check=True, capture_output=True)
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True, capture_output=True,
                             text=True).stdout.strip()
    code = ("import sys, pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_oracle_pins.py']))\n")
    r = run_child(code, {"LD_PRELOAD": runtime, "MOE_ORACLE_LIB": lib, "ASAN_OPTIONS": ASAN_OPTIONS,
                         "UBSAN_OPTIONS": UBSAN_OPTIONS})
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert " passed" in r.stdout and "failed" not in r.stdout
