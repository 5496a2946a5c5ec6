"""Compile the HIP library in-tree for gfx950.

``python -m rvq_codebook_code_amd.build`` (or ``build()``) runs hipcc on
``csrc/qp.hip`` and writes ``rvq_codebook_code_amd/libqp.so``; on the same
source with ``QP_TIMELINE`` defined for ``libqp_timeline.so`` (the dataflow
kernels stamp each phase's start, staged inputs and end into the taps buffer,
the batched path's kernels their start, K-loop end and end into a device
array; ``bench.py --timeline`` reads them); and on ``csrc/probe_mfma.hip``,
``csrc/probe_exchange.hip`` and ``csrc/probe_boundary.hip`` (the matrix-core
peak, record hand-off and kernel-boundary probes bench.py can run) for
``libqp_probe.so``.  The three compile in parallel.
hipcc cross-compiles without a GPU.
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
TIMELINE_LIB = os.path.join(PKG, "libqp_timeline.so")


def _start(srcs, out: str, extra, verbose: bool):
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, f"-I{INCLUDE}", f"-I{CSRC}", *srcs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def build(verbose: bool = False) -> str:
    """The library (libqp.so), its timeline build (libqp_timeline.so) and the
    probes (libqp_probe.so), compiled in parallel."""
    jobs = [
        (LIB, _start([os.path.join(CSRC, "qp.hip")], LIB, [], verbose)),
        (TIMELINE_LIB, _start([os.path.join(CSRC, "qp.hip")], TIMELINE_LIB, ["-DQP_TIMELINE"], verbose)),
        (PROBE_LIB, _start([os.path.join(CSRC, "probe_mfma.hip"), os.path.join(CSRC, "probe_exchange.hip"),
                            os.path.join(CSRC, "probe_boundary.hip")],
                           PROBE_LIB, [], verbose)),
    ]
    failed = []
    for out, proc in jobs:
        log, _ = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(log)
            failed.append((os.path.basename(out), proc.returncode))
        else:
            os.replace(out + ".tmp", out)
    if failed:
        raise RuntimeError(f"hipcc failed: {failed}")
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
