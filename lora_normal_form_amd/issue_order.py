"""Check the load issue order the decode main kernel's counted waits rely on.

k_decode_main waits for a ring stage with `s_waitcnt vmcnt(n)`, where n is
the number of loads the wave issued after that stage's rows and W. The count
holds only if, in every step of the K loop, the stage's direct-to-LDS row
loads are issued before the next stage's W loads (a W load moved above a row
load leaves that row load uncounted, and the stage is read before it lands).
This compiles decode.hip's device code to AMDGPU assembly and checks the
order in every instantiation of the kernel. Run it after changing the K loop:

    python -m lora_normal_form_amd.issue_order      (exit status 1 on a violation)
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

from . import build


def kernel_steps(asm: str):
    """{kernel symbol: [ops of each step between barriers]} for k_decode_main."""
    lines = asm.split("\n")
    out = {}
    for i, line in enumerate(lines):
        if not re.match(r"^_ZN5scute13k_decode_main.*:", line):
            continue
        name = line.split(":")[0]
        steps, cur = [], []
        for body in lines[i + 1:]:
            if body.startswith(".Lfunc_end"):
                break
            m = re.search(r"\b(buffer_load_dwordx4|global_load_lds_dwordx4|s_barrier)\b", body)
            if not m:
                continue
            if m.group(1) == "s_barrier":
                steps.append(cur)
                cur = []
            else:
                cur.append(m.group(1))
        out[name] = steps
    return out


def violations(asm: str):
    """(kernel, step index) of every step where a row load follows a W load."""
    bad = []
    for name, steps in kernel_steps(asm).items():
        for j, ops in enumerate(steps[1:], 1):
            seen_w = False
            for o in ops:
                if o == "buffer_load_dwordx4":
                    seen_w = True
                elif seen_w:
                    bad.append((name, j))
                    break
    return bad


def main() -> int:
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "decode.s")
        cmd = [build.HIPCC] + build.COMMON + build.HIP_FLAGS + [
            "--cuda-device-only", "-S", "-o", out, os.path.join(build.CSRC, "decode.hip")]
        subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        asm = open(out).read()
    steps = kernel_steps(asm)
    bad = violations(asm)
    for name, j in bad:
        print(f"row load after a W load: {name} step {j}")
    print(f"{len(steps)} kernels, {sum(len(s) for s in steps.values())} steps, {len(bad)} violations")
    return 1 if bad or not steps else 0


if __name__ == "__main__":
    sys.exit(main())
