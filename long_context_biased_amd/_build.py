"""Build libabg.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libabg.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["biased_mqa_fwd.hip", "pair_bias_project.hip", "scratch.hip", "abg_api.cpp"]

# Packed FP32 VALU instructions are disabled for all device code (the
# compiler would otherwise form v_pk_* from ordinary float code).
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature: drop that noise.
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError("command failed:\n  " + " ".join(cmd) + "\n" + out)
    return out


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source and link ``libabg.so`` next to this file.

    Always recompiles (the caller asked for a build).  Returns the library
    path.  The output is written to a temporary name and renamed, so a running
    process that has the old library loaded is not disturbed.
    """
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    flags = HIP_FLAGS + list(extra_flags or [])

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        out = _run(cmd)
        if verbose and out.strip():
            print(out, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
