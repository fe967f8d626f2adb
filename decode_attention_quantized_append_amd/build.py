"""Build the HIP library (libkvq.so, gfx950), its CPU twin for host-logic
tests (libkvq_nodev.so) and the benchmark's streaming-read probe
(libkvq_probe.so), in-tree next to the sources.

    python -m decode_attention_quantized_append_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libkvq.so")
LIB_NODEV = os.path.join(PKG, "libkvq_nodev.so")
LIB_PROBE = os.path.join(PKG, "libkvq_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: no packed fp32 VALU instructions are generated.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-I", INCLUDE]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_hip(verbose: bool = True) -> str:
    srcs = [os.path.join(CSRC, "kvq_host.cpp"), os.path.join(CSRC, "kvq_kernels.hip")]
    tmp = LIB + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", "-o", tmp, *srcs], verbose)
    os.replace(tmp, LIB)
    return LIB


def build_nodev(verbose: bool = True) -> str:
    srcs = [os.path.join(CSRC, "kvq_host.cpp"), os.path.join(CSRC, "kvq_nodev.cpp")]
    tmp = LIB_NODEV + ".tmp"
    _run(["g++", *CXX_FLAGS, "-shared", "-o", tmp, *srcs], verbose)
    os.replace(tmp, LIB_NODEV)
    return LIB_NODEV


def build_probe(verbose: bool = True) -> str:
    tmp = LIB_PROBE + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-shared", "-o", tmp, os.path.join(CSRC, "kvq_probe.hip")], verbose)
    os.replace(tmp, LIB_PROBE)
    return LIB_PROBE


def build_all(verbose: bool = True):
    return build_hip(verbose), build_nodev(verbose), build_probe(verbose)


if __name__ == "__main__":
    build_all(verbose="-q" not in sys.argv)
