"""Compile libeq.so in-tree for gfx950.

host_codec.cpp is plain C++17 (g++); decode.hip is HIP for gfx950 only
(wave64, CDNA4), built without packed-fp32 instruction selection.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libeq.so")
ARCH = os.environ.get("EQ_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wall", "-Wno-unused-command-line-argument"]


def _run(cmd, verbose):
    if verbose:
        print("+", " ".join(cmd), flush=True)
    subprocess.check_call(cmd, cwd=ROOT)


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    host_o = os.path.join(BUILD, "host_codec.o")
    dev_o = os.path.join(BUILD, "decode.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-pthread", "-Wall", "-Wextra",
          "-c", os.path.join(CSRC, "host_codec.cpp"), "-o", host_o], verbose)
    _run(["hipcc", *HIPCC_FLAGS, "-c", os.path.join(CSRC, "decode.hip"), "-o", dev_o], verbose)
    tmp = LIB + ".tmp"
    _run(["hipcc", "-shared", f"--offload-arch={ARCH}", host_o, dev_o, "-o", tmp, "-pthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
