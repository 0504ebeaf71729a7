"""Host-only run of the CPU test suite under AddressSanitizer and
UndefinedBehaviorSanitizer.

Builds libscute_san.so (``build(sanitize=True)``: the host side of every
source instrumented, device code untouched), then runs ``pytest -m "not
gpu"`` with the sanitizer runtime preloaded into the (uninstrumented) Python
interpreter and SCUTE_LIB pointing the binding at the sanitized library.
Leak checking is off (the interpreter's own allocations would swamp it); any
sanitizer report stops the run with a non-zero status.

    python -m lora_normal_form_amd.sanitize_check [--no-build] [pytest args...]
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

from . import build as B


def asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's AddressSanitizer runtime was not found under /opt/rocm/lib/llvm")
    return hits[-1]


def main(argv=None) -> int:
    argv = list(sys.argv[1:] if argv is None else argv)
    if "--no-build" in argv:
        argv.remove("--no-build")
    else:
        B.build(verbose=True, sanitize=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["SCUTE_LIB"] = B.LIB_SAN
    cmd = [sys.executable, "-m", "pytest", os.path.join(B.ROOT, "tests"), "-m", "not gpu", "-q",
           "-p", "no:cacheprovider"] + argv
    print("sanitize_check: " + " ".join(cmd), flush=True)
    return subprocess.call(cmd, cwd=B.ROOT, env=env)


if __name__ == "__main__":
    sys.exit(main())
