"""Compile libeq.so in-tree for gfx950.

host_codec.cpp is plain C++17 (g++); decode.hip and encode.hip are HIP for
gfx950 only (wave64, CDNA4), built without packed-fp32 instruction
selection; pipeline.hip is the host-side block schedule.
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


def build_library(verbose: bool = False, out: str = LIB, defines: dict | None = None,
                  build_dir: str = BUILD) -> str:
    """Build libeq.so (or a variant with extra -D defines at `out`)."""
    os.makedirs(build_dir, exist_ok=True)
    host_o = os.path.join(build_dir, "host_codec.o")
    dev_o = os.path.join(build_dir, "decode.o")
    dflags = [f"-D{k}={v}" for k, v in (defines or {}).items()]
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-pthread", "-Wall", "-Wextra",
          "-c", os.path.join(CSRC, "host_codec.cpp"), "-o", host_o], verbose)
    enc_o = os.path.join(build_dir, "encode.o")
    _run(["hipcc", *HIPCC_FLAGS, *dflags, "-c", os.path.join(CSRC, "decode.hip"), "-o", dev_o], verbose)
    _run(["hipcc", *HIPCC_FLAGS, *dflags, "-c", os.path.join(CSRC, "encode.hip"), "-o", enc_o], verbose)
    pipe_o = os.path.join(build_dir, "pipeline.o")
    _run(["hipcc", *HIPCC_FLAGS, "-c", os.path.join(CSRC, "pipeline.hip"), "-o", pipe_o], verbose)
    tmp = out + ".tmp"
    _run(["hipcc", "-shared", f"--offload-arch={ARCH}", host_o, dev_o, enc_o, pipe_o, "-o", tmp, "-pthread"],
         verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build_library(verbose=True)
