"""Sanitizer builds on the CPU (no GPU): the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer, driven through every function; and the C ABI's
host-side argument checks built with host-only sanitizers, driven through every
rejection path (the kernel launchers are stubs that abort, so any call that
slipped past the checks would fail the test)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "trellis_quantized_moe_exl3_amd", "csrc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"], tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0 and "oracle driver: ok" in r.stdout, r.stdout + r.stderr


def _launcher_stubs():
    """Definitions that abort for every launcher internal.h declares."""
    text = open(os.path.join(CSRC, "internal.h")).read()
    decls = re.findall(r"^hipError_t (launch_\w+\([^;]*\));", text, re.M)
    assert len(decls) >= 20
    body = "\n".join(f"hipError_t {d} {{ abort(); }}" for d in decls)
    return f'#include <stdlib.h>\n#include "internal.h"\nnamespace moe {{\n{body}\n}}\n'


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_abi_host_checks_under_sanitizers(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    obj = str(tmp_path / "moe_exl3.o")
    _run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-x", "hip",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-c", os.path.join(CSRC, "moe_exl3.cpp"), "-o", obj], tmp_path)
    stubs = tmp_path / "stubs.cpp"
    stubs.write_text(_launcher_stubs())
    exe = str(tmp_path / "abi_asan")
    cxx = shutil.which("g++")
    # the host files include hip_runtime.h, so the host compiler sees the HIP
    # headers through ROCm's clang
    clang = "/opt/rocm/llvm/bin/clang++"
    _run([clang, "-O1", "-g", "-std=c++17", "-x", "hip", "--cuda-host-only", "-fsanitize=address,undefined",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", str(stubs), "-o",
          str(tmp_path / "stubs.o")], tmp_path)
    _run([cxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_driver.cpp"), obj, str(tmp_path / "stubs.o"),
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe], tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, env=SAN_ENV)
    assert r.returncode == 0 and "abi driver: ok" in r.stdout, r.stdout + r.stderr
