"""Build the HIP library ``libtm.so`` in-tree for gfx950 with hipcc.

Each source compiles to its own object (in parallel, under ``_build/`` at the
repository root), then one hipcc line links the shared library.  No source
calls device code of another, so no relocatable device code is needed.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("tm_kernels.hip", "tm_r3.hip", "tm_retrieve.hip", "tm_project.hip",
                                           "tm_mac.hip", "tm_bwd.hip", "tm_api.hip")]
HEADERS = [os.path.join(CSRC, "tm_internal.h"), os.path.join(CSRC, "tm_device.h"), os.path.join(ROOT, "include", "tm.h")]
LIB = os.path.join(HERE, "libtm.so")
OBJDIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    errs = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    return res.returncode, errs


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.basename(s) + ".%d.o" % os.getpid()) for s in SOURCES]
    cmds = [[HIPCC] + FLAGS + ["-I" + os.path.join(ROOT, "include"), "-c", "-o", o, s]
            for s, o in zip(SOURCES, objs)]
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for cmd, (rc, errs) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if errs and (rc != 0 or verbose):
            sys.stderr.write("\n".join(errs) + "\n")
        failed |= rc != 0
    tmp = LIB + ".tmp%d" % os.getpid()
    try:
        if failed:
            raise RuntimeError("hipcc failed")
        rc, errs = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
        if rc != 0:
            sys.stderr.write("\n".join(errs) + "\n")
            raise RuntimeError("hipcc link failed (%d)" % rc)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
