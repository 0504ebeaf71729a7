"""Build libscute.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); host sources are
plain C++17 compiled by hipcc's host pass.

``build(sanitize=True)`` (``python -m lora_normal_form_amd.build --sanitize``)
builds libscute_san.so instead: the host side of every source with
AddressSanitizer and UndefinedBehaviorSanitizer (``-Xarch_host`` in front of
each ``-fsanitize=``, so no device code is instrumented), for host-only runs
(``python -m lora_normal_form_amd.sanitize_check``).
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
BUILD_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(PKG, "libscute_san.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined"]
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


def build(verbose: bool = False, jobs: int = 8, sanitize: bool = False) -> str:
    """Compile every source and link libscute.so (libscute_san.so with
    sanitize). Returns the library path."""
    bdir, lib = (BUILD_SAN, LIB_SAN) if sanitize else (BUILD, LIB)
    os.makedirs(bdir, exist_ok=True)
    t0 = time.time()
    cmds, objs = [], []
    for src in HOST_SRCS + HIP_SRCS:
        obj = os.path.join(bdir, src + ".o")
        flags = COMMON + (HIP_FLAGS if src.endswith(".hip") else []) + (SAN_FLAGS if sanitize else [])
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
    tmp = lib + ".tmp"
    link = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-shared-libasan"] if sanitize else []
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + link + objs)
    os.replace(tmp, lib)
    if verbose:
        sys.stderr.write(f"built {lib} in {time.time() - t0:.1f}s\n")
    return lib


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
