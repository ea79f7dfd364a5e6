"""Compile libsiggate.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m sigmoid_group_limited_amd.build
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
LIBRARY = os.path.join(PKG, "libsiggate.so")
# exports only the siggate_* functions
VERSION_SCRIPT = os.path.join(CSRC, "siggate.map")
EXAMPLE_SOURCE = os.path.join(PKG, "examples", "route_c.cpp")
EXAMPLE = os.path.join(PKG, "route_c")
SOURCES = ["gate.hip", "logits_x3.hip", "dispatch.hip", "combine.hip", "ep.hip", "api.hip"]
ARCH = "gfx950"

# Packed fp32 arithmetic is switched off for all device code.  Symbols are
# hidden by default: the library exports only the C ABI of siggate.h.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
               "-Wall", "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def build(verbose: bool = False) -> str:
    """Compile every HIP source into ``libsiggate.so`` next to this file."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs,
           f"-Wl,--version-script={VERSION_SCRIPT}", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIBRARY)
    build_example(verbose)
    return LIBRARY


def build_example(verbose: bool = False) -> str:
    """Compile the C ABI example (host code only) against the library."""
    flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [hipcc(), *flags, "-I", INCLUDE, EXAMPLE_SOURCE, "-L", PKG, "-lsiggate",
           "-Wl,-rpath,$ORIGIN", "-o", EXAMPLE]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on the example:\n" + "\n".join(msgs))
    return EXAMPLE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
