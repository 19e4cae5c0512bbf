"""Builds libmonolayer.so (HIP for gfx950) in-tree with hipcc."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmonolayer.so")
ARCH = os.environ.get("MONO_OFFLOAD_ARCH", "gfx950")

# Packed-FP32 instructions are disabled for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
             "-Wno-unused-but-set-variable"]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False, extra=()) -> str:
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-shared", "-o", LIB + ".tmp",
           os.path.join(CSRC, "mono_device.hip"), os.path.join(CSRC, "mono_api.cpp")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("libmonolayer build failed:\n" + " ".join(cmd) + "\n" + msgs)
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
