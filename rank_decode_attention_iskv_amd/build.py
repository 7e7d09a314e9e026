"""Build libiskv.so (HIP kernels for gfx950 + the C-ABI host library) in-tree.

    python -m rank_decode_attention_iskv_amd.build

Compiles every source under csrc/ with hipcc for gfx950 and writes
rank_decode_attention_iskv_amd/libiskv.so next to this file.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libiskv.so")

SOURCES = ["iskv.cpp", "maintain.hip", "fold.hip", "decode.hip"]

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    for p in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(p) and os.path.exists(p):
            return p
    return "hipcc"


def build(verbose=False):
    cmd = [hipcc()] + FLAGS + [os.path.join(SRC, s) for s in SOURCES] + ["-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libiskv.so")
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
