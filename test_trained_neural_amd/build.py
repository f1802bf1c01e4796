"""Build the HIP library ``libtm.so`` in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("tm_kernels.hip", "tm_r3.hip", "tm_retrieve.hip", "tm_project.hip", "tm_mac.hip", "tm_api.hip")]
HEADERS = [os.path.join(CSRC, "tm_internal.h"), os.path.join(CSRC, "tm_device.h"), os.path.join(ROOT, "include", "tm.h")]
LIB = os.path.join(HERE, "libtm.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-I" + os.path.join(ROOT, "include"), "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    errs = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(errs) + "\n")
        raise RuntimeError("hipcc failed (%d)" % res.returncode)
    if verbose and errs:
        print("\n".join(errs))
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
