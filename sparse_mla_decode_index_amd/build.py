"""Build libsmd.so in-tree with hipcc for gfx950.

Every HIP translation unit is compiled with packed-FP32 instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass
warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
INCLUDE = PKG.parent / "include"
LIB = PKG / "libsmd.so"
BUILD_DIR = PKG.parent / "_build"

SOURCES = ["api.cpp", "plan.cpp", "noalloc.hip", "decode_kernels.hip", "wide_kernel.hip", "persistent_kernel.hip",
           "writer_kernel.hip", "paged_kernel.hip"]
ARCH = os.environ.get("SMD_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsmd)")


def common_flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> Path:
    cc = hipcc()
    BUILD_DIR.mkdir(exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:  # the translation units compile in parallel
        obj = BUILD_DIR / (Path(src).stem + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *common_flags(), "-c", *lang, str(CSRC / src), "-o", str(obj)]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(str(obj))
    failed = []
    for src, proc in procs:
        out, _ = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(out)
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc link of libsmd.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
