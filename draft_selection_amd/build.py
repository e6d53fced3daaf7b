"""Build libdsel.so in-tree with hipcc for gfx950 (no torch involved)."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SO = os.path.join(PKG, "libdsel.so")
SRC = os.path.join(PKG, "csrc", "libdsel.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
]


def build(verbose: bool = False) -> str:
    tmp = SO + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to build libdsel.so")
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
