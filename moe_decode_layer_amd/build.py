"""Builds libmonolayer.so (HIP for gfx950) in-tree with hipcc, one object per source in
parallel, then links them."""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmonolayer.so")
ARCH = os.environ.get("MONO_OFFLOAD_ARCH", "gfx950")
SOURCES = ["mono_launch.hip", "mono_k_f32.hip", "mono_k_bf16.hip", "mono_k_q8.hip",
           "mono_k_fp4.hip", "mono_api.cpp", "mono_static.hip", "mono_head.hip"]

# Packed-FP32 instructions are disabled for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
             "-Wno-unused-but-set-variable"]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, msgs, cmd


def build(verbose: bool = False, extra=(), jobs: int = 0) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        cmds.append([hipcc(), *HIP_FLAGS, *extra, "-c", "-o", obj, os.path.join(CSRC, src)])
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for rc, msgs, cmd in results:
        if rc != 0:
            raise RuntimeError("libmonolayer build failed:\n" + " ".join(cmd) + "\n" + msgs)
        if verbose and msgs.strip():
            print(msgs, file=sys.stderr)
    objs = [c[c.index("-o") + 1] for c in cmds]
    rc, msgs, cmd = _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-o", LIB + ".tmp", *objs])
    if rc != 0:
        raise RuntimeError("libmonolayer link failed:\n" + " ".join(cmd) + "\n" + msgs)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
