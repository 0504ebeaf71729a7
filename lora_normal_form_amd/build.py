"""Build libscute.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); host sources are
plain C++17 compiled by hipcc's host pass.
"""

from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libscute.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HOST_SRCS = ["layer.cpp", "plan.cpp", "plan_decode.cpp", "plan_prefill.cpp", "plan_fdecode.cpp"]
HIP_SRCS = ["forward.hip", "decode.hip", "prefill.hip", "fdecode.hip", "rotate.hip", "routes.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include")]
HIP_FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout)
        raise RuntimeError(f"build failed: {os.path.basename(cmd[-1])}")
    return r.stdout


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link libscute.so. Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    cmds, objs = [], []
    for src in HOST_SRCS + HIP_SRCS:
        obj = os.path.join(BUILD, src + ".o")
        flags = COMMON + (HIP_FLAGS if src.endswith(".hip") else [])
        cmds.append([HIPCC] + flags + ["-c", "-o", obj, os.path.join(CSRC, src)])
        objs.append(obj)
    procs = []
    for c in cmds:
        procs.append((c, subprocess.Popen(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                          text=True)))
        while sum(p.poll() is None for _, p in procs) >= jobs:
            time.sleep(0.05)
    failed = False
    for c, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(" ".join(c) + "\n" + out)
            failed = True
        elif verbose and out.strip():
            sys.stderr.write(out)
    if failed:
        raise RuntimeError("libscute build failed")
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if verbose:
        sys.stderr.write(f"built {LIB} in {time.time() - t0:.1f}s\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
