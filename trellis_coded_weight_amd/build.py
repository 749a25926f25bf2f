"""Build the gfx950 encoder library (libexl3_gfx950.so) in-tree with hipcc.

Numeric flags: -ffp-contract=off keeps every subtract / multiply / add a
separately rounded binary32 operation (no fused multiply-add), binary32
denormals are kept, and packed-FP32 instructions are switched off.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libexl3_gfx950.so")
OBJ_DIR = os.path.join(HERE, "_build")

SOURCES = ["api.hip", "viterbi_fwd.hip", "viterbi_fwd_f16.hip", "traceback.hip", "regularize.hip",
           "channel.hip", "ldlq.hip", "codebook.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-std=c++17", "-O3", "-fPIC", "--offload-arch=gfx950",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, src + ".o")
        cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
