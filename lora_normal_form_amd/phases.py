"""Phase timestamps of the two-launch decode main kernel.

Builds an instrumented copy of the library in which thread 0 of every
work-group of k_decode_main writes the 100 MHz real-time counter
(s_memrealtime) at each phase boundary; nothing else changes, so the copy
computes the same results. Then runs named workloads through it (on the two-launch decode path: SCUTE_DECODE=2) and prints,
per phase, the median over work-groups of the time since the earliest
work-group started (medians of five forwards):

    start          the work-group begins
    stage0 data    the first ring stage has landed (after its barrier)
    kloop end      the K loop's last MFMAs are issued and every load landed
    meet           the K halves have met in LDS
    expand done    row pass 1, the expand and the dense VeRA product are done
    before stores  row pass 2 is done (y or the slice tile is stored next)
    arrived        this slice has stored its tile and counted its arrival
    last done      the last slice of a tile has stored y

    python -m lora_normal_form_amd.phases build [DIR]      (compile; no GPU needed)
    python -m lora_normal_form_amd.phases run [DIR] 2 3    (workload indices; one GPU)

DIR defaults to lora_normal_form_amd/_phases.
"""

from __future__ import annotations

import ctypes
import importlib
import importlib.util
import os
import shutil
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
DEFAULT_DIR = os.path.join(PKG, "_phases")
NAMES = ["start", "stage0 data", "kloop end", "meet", "expand done", "before stores", "arrived",
         "last done"]
SLOTS = 8192 * 8


def _patch(src: str) -> str:
    def rep(s, a, b):
        if s.count(a) != 1:
            raise RuntimeError(f"instrumentation anchor not found once: {a[:60]!r}")
        return s.replace(a, b)
    s = rep(src, "namespace scute {\n", """namespace scute {
__device__ unsigned long long g_phase_stamps[8192 * 8];
__device__ __forceinline__ void phase_stamp(int i) {
  if (threadIdx.x == 0)
    g_phase_stamps[(blockIdx.y * gridDim.x + blockIdx.x) * 8 + i] = __builtin_amdgcn_s_memrealtime();
}
""")
    s = rep(s, "  const int m = lane & 31, h = lane >> 5;\n  const int cb = wave & 1, kp = wave >> 1;\n  const int mgx",
            "  const int m = lane & 31, h = lane >> 5;\n  phase_stamp(0);\n  const int cb = wave & 1, kp = wave >> 1;\n  const int mgx")
    s = rep(s, "    if (tid < MGT) vflag[tid] = 0;\n", "    if (tid < MGT) vflag[tid] = 0;\n    phase_stamp(1);\n")
    s = rep(s, "  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // clamped tail prefetches\n  wg_barrier();\n",
            "  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // clamped tail prefetches\n  wg_barrier();\n  phase_stamp(2);\n")
    s = rep(s, "  lds_barrier();  // other waves read these LDS writes next\n",
            "  lds_barrier();  // other waves read these LDS writes next\n  phase_stamp(3);\n")
    s = rep(s, "  if (a.gv1 > a.gv0) dense_vera<MGT>(a, V, vflag, kc, cb, kp, tid, m, h, ncol);\n  lds_barrier();\n",
            "  if (a.gv1 > a.gv0) dense_vera<MGT>(a, V, vflag, kc, cb, kp, tid, m, h, ncol);\n  lds_barrier();\n  phase_stamp(4);\n")
    s = rep(s, "  if (a.S == 1) {\n", "  phase_stamp(5);\n  if (a.S == 1) {\n")
    s = rep(s, "  lds_barrier();  // last_flag is read by every wave\n  if (!last_flag) return;\n",
            "  lds_barrier();  // last_flag is read by every wave\n  phase_stamp(6);\n  if (!last_flag) return;\n")
    i = s.index("      if (tk >= 0) stg4(a.y + (size_t)tk * a.d_out + cbase, tot[j]);")
    j = s.index("\n}\n", i)
    s = s[:j] + "\n  wait_vm_all();\n  phase_stamp(7);" + s[j:]
    return s + """
extern "C" int scute_phase_clear() {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scute::g_phase_stamps)) != hipSuccess) return -1;
  return (int)hipMemset(p, 0, sizeof(unsigned long long) * 8192 * 8);
}
extern "C" int scute_phase_read(unsigned long long* out, int n) {
  return (int)hipMemcpyFromSymbol(out, HIP_SYMBOL(scute::g_phase_stamps), sizeof(unsigned long long) * n);
}
"""


def build(dest: str = DEFAULT_DIR) -> str:
    """Copy the package and its header to dest, instrument decode.hip, build."""
    pkg = os.path.join(dest, "lora_normal_form_amd")
    if os.path.exists(pkg):
        shutil.rmtree(pkg)
    os.makedirs(os.path.join(dest, "include"), exist_ok=True)
    shutil.copy(os.path.join(ROOT, "include", "scute.h"), os.path.join(dest, "include", "scute.h"))
    shutil.copytree(PKG, pkg, ignore=shutil.ignore_patterns("_build", "_build_san", "_phases", "*.so",
                                                            "__pycache__"))
    p = os.path.join(pkg, "csrc", "decode.hip")
    with open(p) as f:
        src = f.read()
    with open(p, "w") as f:
        f.write(_patch(src))
    spec = importlib.util.spec_from_file_location("_scute_phases_build", os.path.join(pkg, "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b.build(verbose=False)


def run(dest: str, workloads) -> None:
    lib_path = os.path.join(dest, "lora_normal_form_amd", "libscute.so")
    if not os.path.exists(lib_path):
        raise SystemExit(f"{lib_path} missing: run `build` first")
    os.environ["SCUTE_LIB"] = lib_path
    # the stamps are in the two-launch decode kernel: plan every batch there
    os.environ["SCUTE_DECODE"] = "2"
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    from synth import make_config
    from . import scute, workload as glue
    if scute.LIB_PATH != lib_path:
        raise SystemExit("the instrumented library is not the one loaded")
    lib = ctypes.CDLL(lib_path)
    for widx in workloads:
        wl = make_config(widx)
        ld = glue.load(wl, device=0)
        for _ in range(5):
            ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
        torch.cuda.synchronize()
        runs = []
        for _ in range(5):
            lib.scute_phase_clear()
            torch.cuda.synchronize()
            ld.layer.forward(ld.batch, ld.x, ld.W, ld.y)
            torch.cuda.synchronize()
            buf = (ctypes.c_ulonglong * SLOTS)()
            lib.scute_phase_read(buf, SLOTS)
            a = np.frombuffer(buf, dtype=np.uint64).reshape(-1, 8).astype(np.int64)
            runs.append(a[a[:, 0] > 0])
        print(f"{wl.name}: {len(runs[0])} work-groups of k_decode_main; us since the first started")
        print("| phase | median | min | max |\n|---|---|---|---|")
        for i, nm in enumerate(NAMES):
            med, lo, hi = [], [], []
            for g in runs:
                col = g[:, i][g[:, i] > 0]
                if len(col):
                    col = (col - g[:, 0].min()) / 100.0
                    med.append(np.median(col)); lo.append(col.min()); hi.append(col.max())
            if med:
                print(f"| {nm} | {np.median(med):.2f} | {np.median(lo):.2f} | {np.median(hi):.2f} |")
        ld.batch.close()
        ld.layer.close()


def main(argv=None) -> int:
    argv = list(sys.argv[1:] if argv is None else argv)
    if not argv or argv[0] not in ("build", "run"):
        print(__doc__)
        return 2
    cmd, rest = argv[0], argv[1:]
    dest = rest.pop(0) if rest and not rest[0].isdigit() else DEFAULT_DIR
    if cmd == "build":
        print(build(os.path.abspath(dest)))
    else:
        run(os.path.abspath(dest), [int(a) for a in rest] or [2])
    return 0


if __name__ == "__main__":
    sys.exit(main())
