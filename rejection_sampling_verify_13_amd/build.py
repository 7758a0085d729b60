"""Compile the HIP library for gfx950 into this package directory."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "spec_verify.hip")
LIB = os.path.join(HERE, "libspecverify.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # packed fp32 instructions stay disabled: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


EXAMPLE_SRC = os.path.join(HERE, "examples", "verify_from_c.c")
EXAMPLE = os.path.join(HERE, "verify_from_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed for " + SRC)
    os.replace(tmp, LIB)
    build_example(verbose)
    return LIB


def build_example(verbose: bool = False) -> str:
    """The plain-C caller of the library (a host program: gcc and the HIP runtime)."""
    tmp = EXAMPLE + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O2", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), EXAMPLE_SRC, "-L", HERE, "-lspecverify",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("gcc failed for " + EXAMPLE_SRC)
    os.replace(tmp, EXAMPLE)
    return EXAMPLE


if __name__ == "__main__":
    print(build(verbose=True))
