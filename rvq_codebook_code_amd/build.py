"""Compile the HIP library in-tree for gfx950.

``python -m rvq_codebook_code_amd.build`` (or ``build()``) runs hipcc on
``csrc/qp.hip`` and writes ``rvq_codebook_code_amd/libqp.so``, and on
``csrc/probe_mfma.hip`` and ``csrc/probe_exchange.hip`` (the matrix-core
peak and record hand-off probes bench.py can run) for ``libqp_probe.so``.  hipcc cross-compiles without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqp.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-command-line-argument",
    # packed fp32 arithmetic stays off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the library)")


PROBE_LIB = os.path.join(PKG, "libqp_probe.so")


def _hipcc(src: str, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, out)


def _hipcc_many(srcs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """The library (libqp.so) and the matrix-core peak probe (libqp_probe.so)."""
    _hipcc(os.path.join(CSRC, "qp.hip"), LIB, verbose)
    _hipcc_many([os.path.join(CSRC, "probe_mfma.hip"), os.path.join(CSRC, "probe_exchange.hip")], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
