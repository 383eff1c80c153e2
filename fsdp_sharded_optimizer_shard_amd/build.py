"""Build libzeroshard.so for gfx950 with hipcc, in-tree.

Flags:
  --offload-arch=gfx950           CDNA4 only; no other target is built.
  -ffp-contract=off               no multiply-add fusion (each operation
                                  rounds once, as the arithmetic contract
                                  of the header states).
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                  keep the compiler from forming packed fp32
                                  (v_pk_*_f32) instructions.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libzeroshard.so")
SOURCES = [os.path.join(CSRC, "layout.cpp"), os.path.join(CSRC, "kernels.hip"),
           os.path.join(CSRC, "sweep.cpp"), os.path.join(CSRC, "gemm.hip"),
           os.path.join(CSRC, "linear.cpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", f"-I{INCLUDE}"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libzeroshard.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
