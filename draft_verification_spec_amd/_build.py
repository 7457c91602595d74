"""Compile the HIP library for gfx950 in-tree (libspec_verify.so next to this file):
the verification kernel and the distillation kernel."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "spec_verify.hip")
SRCS = [SRC, os.path.join(HERE, "csrc", "sv_kd.hip")]
LIB = os.path.join(HERE, "libspec_verify.so")
HEADER = os.path.join(ROOT, "include", "spec_verify.h")
# the benchmark's stream-read reference (measurement only; not part of the library)
STREAM_SRC = os.path.join(HERE, "csrc", "sv_stream_read.hip")
STREAM_LIB = os.path.join(HERE, "libsv_stream_read.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                                   # identical arithmetic wherever a formula repeats
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc(srcs, out, verbose, extra=()):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)


def build(verbose: bool = False, extra=()) -> str:
    _hipcc(SRCS, LIB, verbose, extra)
    _hipcc([STREAM_SRC], STREAM_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
