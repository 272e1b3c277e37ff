"""Compile libfavor.so (HIP for gfx950) in-tree with hipcc.

Every .hip / .cpp file under csrc/ is compiled to an object under _build/ (in
parallel) and linked into kernelized_linear_attention_favor_amd/libfavor.so.
The instruction-rate probes under ubench/ (used by bench.py's measurements,
not part of the attention library) go into libfavor_ubench.so beside it.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfavor.so")
UBENCH = os.path.join(PKG, "ubench")
UBENCH_LIB = os.path.join(PKG, "libfavor_ubench.so")

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-function",
    # keep packed fp32 VALU forms out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *CFLAGS, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), *CFLAGS, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    usrcs = sorted(glob.glob(os.path.join(UBENCH, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(usrcs))) as ex:
        objs = list(ex.map(_compile, srcs + usrcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], UBENCH_LIB)
    if verbose:
        print(f"built {LIB} and {UBENCH_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
