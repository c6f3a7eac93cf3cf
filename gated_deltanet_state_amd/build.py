"""Build libgdn.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
SOURCES = ["gdn_api.cpp", "gdn_decode.hip", "gdn_chunk_valu.hip", "gdn_chunk_mfma.hip", "kda_chunk_mfma.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions stay off: only scalar fp32 VALU code is generated
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = ["hipcc", *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    subprocess.run(cmd, check=True)


def build(verbose: bool = True, jobs: int = 4) -> str:
    """Compile every source (in parallel) and link libgdn.so next to this file."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    t0 = time.time()
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    procs = []
    for src, obj in zip(SOURCES, objs):
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = ["hipcc", *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd)))
        while sum(p.poll() is None for _, p in procs) >= jobs:
            time.sleep(0.05)
    failed = [s for s, p in procs if p.wait() != 0]
    if failed:
        raise RuntimeError(f"hipcc failed for: {failed}")
    tmp = LIB + ".tmp"
    subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
