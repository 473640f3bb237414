"""Builds libbitnet_w2a8.so in-tree for gfx950 with hipcc.

Usage: python -m bit_gemv_i2_amd.build   (or __graft_entry__.build())
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libbitnet_w2a8.so")
SOURCES = [os.path.join(CSRC, "bitnet_w2a8.hip"), os.path.join(CSRC, "pack.cpp"), os.path.join(CSRC, "probe.hip"),
           os.path.join(CSRC, "gemv_lut.hip")]
HEADERS = [os.path.join(INCLUDE, "bitnet_w2a8.h"), os.path.join(CSRC, "layout.h")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    objs = []
    common = ["-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC, "-Wall"]
    # Packed fp32 VALU instructions stay off in device code.
    dev = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [hipcc()] + common + (dev if src.endswith(".hip") else []) + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.check_call(cmd)
        objs.append(obj)
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
