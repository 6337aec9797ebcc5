"""Compile the HIP library (libqli.so) in-tree for gfx950.

    python -m sparse_attention_token_paged_amd.build

hipcc cross-compiles without a GPU.  All HIP code is built with packed-FP32
instructions disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libqli.so")
SOURCES = [os.path.join(CSRC, f) for f in ("qli_api.cpp", "qli_kernels.hip", "qli_quant.hip",
                                          "qli_attention.hip")]
HEADERS = [os.path.join(CSRC, "qli_internal.h"), os.path.join(INCLUDE, "qli.h")]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def command(out: str) -> list:
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fvisibility=hidden", "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", INCLUDE, "-x", "hip"] + SOURCES + ["-o", out]


def build(verbose: bool = False) -> str:
    """Always recompiles; writes the library atomically."""
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msgs)
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def stale() -> bool:
    if not os.path.exists(LIBRARY):
        return True
    t = os.path.getmtime(LIBRARY)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
