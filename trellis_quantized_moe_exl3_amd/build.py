"""Build libmoe_exl3.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m trellis_quantized_moe_exl3_amd.build

Every source is compiled for gfx950 only.  Packed-fp32 VALU instructions are
disabled (`-packed-fp32-ops`): the fp32 arithmetic here is scalar by design.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe_exl3.so")
SOURCES = ["route.hip", "decode.hip", "gemv.hip", "mfma.hip", "mfma8.hip", "combine.hip", "moe_exl3.cpp"]
# the benchmark's streaming-read probe (achievable HBM bandwidth), a library of its own
BW_SOURCE = "bw_probe.hip"
BW_LIB = os.path.join(HERE, "libmoe_exl3_bw.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-x", "hip",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link the shared library."""
    cc = hipcc()
    tmpdir = tempfile.mkdtemp(prefix="moe_exl3_build_")
    try:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src.rsplit(".", 1)[0] + ".o")
            cmd = [cc, *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
            if p.returncode != 0:
                failed.append((src, text))
            elif verbose and text.strip():
                print(text)
        if failed:
            msg = "\n".join(f"--- {s}\n{t}" for s, t in failed)
            raise RuntimeError(f"hipcc failed:\n{msg}")
        tmp_lib = LIB + ".tmp"
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp_lib]
        subprocess.check_call(cmd)
        os.replace(tmp_lib, LIB)
        tmp_bw = BW_LIB + ".tmp"
        subprocess.check_call([cc, *flags(), "-shared", os.path.join(CSRC, BW_SOURCE), "-o", tmp_bw],
                              stderr=subprocess.DEVNULL if not verbose else None)
        os.replace(tmp_bw, BW_LIB)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
