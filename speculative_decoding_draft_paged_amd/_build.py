"""Build libblockattn.so in-tree with hipcc for gfx950 (no JIT, no torch extension).

The translation units compile in parallel to objects in a temporary folder, then
link into the shared library."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libblockattn.so")

SOURCES = ["api.cpp", "kernels_bf16.hip", "kernels_fp8.hip", "stream_read.hip"]
HEADERS = ["internal.h", "attention_kernels.h"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Packed fp32 VALU forms stay off: ordinary float code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    out_tmp = LIB_PATH + ".tmp"
    tmp = tempfile.mkdtemp(prefix="blockattn_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd)))
            objs.append(obj)
        failed = [src for src, p in procs if p.wait() != 0]
        if failed:
            raise subprocess.CalledProcessError(1, f"hipcc {' '.join(failed)}")
        link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out_tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    os.replace(out_tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
