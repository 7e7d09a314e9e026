"""Build libiskv.so (HIP kernels for gfx950 + the C-ABI host library) in-tree.

    python -m rank_decode_attention_iskv_amd.build

Compiles every source under csrc/ with hipcc for gfx950 (one process per
source, in parallel, into _build/) and links
rank_decode_attention_iskv_amd/libiskv.so next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
OUT = os.path.join(HERE, "libiskv.so")

SOURCES = ["iskv.cpp", "maintain.hip", "fold.hip", "fold_joint.hip", "decode.hip"]

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    p = "/opt/rocm/bin/hipcc"
    return p if os.path.exists(p) else "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    objs, cmds = [], []
    for s in SOURCES:
        o = os.path.join(OBJ, os.path.splitext(s)[0] + ".o")
        objs.append(o)
        cmds.append([hipcc()] + FLAGS + ["-c", os.path.join(SRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", OUT + ".tmp"], verbose)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
