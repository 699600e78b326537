"""Builds libgdn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m gateddeltanet_chunked_delta_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_api.cpp", "host_layout.cpp", "prefill.hip", "decode.hip", "measure.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    # no packed fp32 instructions: the compiler may otherwise emit them from plain float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    errs = [ln for ln in r.stderr.splitlines() if "warning" in ln and "packed-fp32-ops" not in ln]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")


def build(verbose: bool = False) -> str:
    """Compiles every source and links libgdn.so; always recompiles."""
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, s + ".o") for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
