"""Builds libpi0x.so (all HIP kernels + the C ABI) for gfx950 with hipcc, in tree."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "pi0x.hip")
LIB = os.path.join(PKG, "libpi0x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off: hipcc must not form v_pk_* fp32 math
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
]


DRIVER_SRC = os.path.join(PKG, "csrc", "denoise_driver.cpp")
DRIVER = os.path.join(PKG, "denoise_driver")


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"{os.path.basename(cmd[0])} failed ({res.returncode}):\n{out}")
    return out


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    out = _run([HIPCC, *FLAGS, SRC, "-o", tmp])
    if verbose and out.strip():
        print(out, file=sys.stderr)
    os.replace(tmp, LIB)
    # the C++ driver of the ABI (host code only), linked against the library beside it
    dtmp = DRIVER + ".tmp"
    out = _run([HIPCC, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"), DRIVER_SRC,
                "-L", PKG, "-lpi0x", "-Wl,-rpath,$ORIGIN", "-o", dtmp])
    if verbose and out.strip():
        print(out, file=sys.stderr)
    os.replace(dtmp, DRIVER)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
