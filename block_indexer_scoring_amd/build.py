"""Build the gfx950 HIP library libqsa.so in-tree with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def command(out: str = LIB, extra=()):
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # Packed fp32 VALU ops are kept out of the generated code.
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # Leading scalar kernel arguments, up to six dwords (the decode's
            # task table pointer; the top-k rows' address and shape), are
            # preloaded into SGPRs at wave launch.
            "-mllvm", "-amdgpu-kernarg-preload-count=6",
            "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
            *extra, *sources(), "-o", out]


def build(out: str = LIB, verbose: bool = False, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
