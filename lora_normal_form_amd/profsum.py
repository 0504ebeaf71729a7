"""Summaries of rocprofv3 output for the layer's kernels.

    python -m lora_normal_form_amd.profsum stats <kernel_stats.csv>
        Markdown table of per-kernel calls / average duration / share.

    python -m lora_normal_form_amd.profsum traffic --fetch <counter_collection.csv>
        --write <counter_collection.csv> --copy-mib N --workload NAME --out <json>
        HBM bytes per dispatch of every kernel from a FETCH_SIZE run and a
        WRITE_SIZE run. The counters report KiB per dispatch; each counter is
        scaled by the factor that maps its reading for a plain device copy of
        N MiB (the runtime's copy kernel, launched by bench.py --calib-copy N)
        to the N MiB it actually read and wrote. The JSON records the SHA-256
        of the kernel sources' code (comments removed), and bench.py uses the
        figures only while that code is unchanged.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))


def kernel_sources():
    """Every source under csrc/ (kernels and the planners that set their
    tile order, split factors and launch shapes), sorted."""
    d = os.path.join(PKG, "csrc")
    return sorted("csrc/" + f for f in os.listdir(d)
                  if f.endswith((".hip", ".h", ".cpp")))


COPY_KERNEL = "__amd_rocclr_copyBuffer"


def strip_comments(src: str) -> str:
    """C++ source without its comments and blank lines, each line's runs of
    blanks collapsed (string and character literals otherwise kept as they
    are), so that edits to comments or layout alone leave the hash of the
    code unchanged."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (" ".join(ln.split()) for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def source_sha() -> str:
    """SHA-256 over the code of every source under csrc/ (kernels and their
    planners), comments removed."""
    h = hashlib.sha256()
    for rel in kernel_sources():
        path = os.path.join(PKG, rel)
        if os.path.exists(path):
            h.update(rel.encode())
            with open(path, encoding="utf-8") as f:
                h.update(strip_comments(f.read()).encode())
    return h.hexdigest()


def _plain(name: str) -> str:
    """Kernel name without its parameter list and anonymous namespaces."""
    return name.replace("(anonymous namespace)::", "").split("(")[0]


def short_name(name: str):
    """The library's name for one of its kernels (the name bench.py and
    scute_profile_read use: "decode_main", "gemm", ...), or None for kernels
    that are not the library's."""
    base = _plain(name)
    if "scute::" not in base:
        return None
    base = base[base.index("scute::") + len("scute::"):].split("<")[0]
    return base[2:] if base.startswith("k_") else base


def stats_table(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    out = ["| kernel | calls | average (us) | share |", "|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"| `{_plain(r['Name'])}` | {r['Calls']} | "
                   f"{float(r['AverageNs']) / 1e3:.2f} | "
                   f"{100.0 * float(r['TotalDurationNs']) / total:.1f}% |")
    return "\n".join(out)


def counter_per_dispatch(path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter (KiB)."""
    per = defaultdict(dict)
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        per[key[0]][key[1]] = per[key[0]].get(key[1], 0.0) + float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def traffic(fetch_csv: str, write_csv: str, copy_mib: float, workload: str) -> dict:
    fetch = counter_per_dispatch(fetch_csv, "FETCH_SIZE")
    write = counter_per_dispatch(write_csv, "WRITE_SIZE")

    def copy_reading(per):
        vals = [v for k, vs in per.items() if COPY_KERNEL in k for v in vs]
        big = [v for v in vals if v > 0.5 * copy_mib * 1024]
        if not big:
            raise SystemExit(f"no {COPY_KERNEL} dispatch near {copy_mib} MiB in the counters")
        return sum(big) / len(big)

    copy_kib = copy_mib * 1024.0
    f_scale = copy_kib / copy_reading(fetch)
    w_scale = copy_kib / copy_reading(write)
    kernels = {}
    for name in sorted(set(fetch) | set(write)):
        k = short_name(name)
        if k is None:
            continue
        fv, wv = fetch.get(name, []), write.get(name, [])
        kernels[k] = {
            "dispatches": max(len(fv), len(wv)),
            "fetch_bytes": (sum(fv) / len(fv)) * f_scale * 1024.0 if fv else None,
            "write_bytes": (sum(wv) / len(wv)) * w_scale * 1024.0 if wv else None,
        }
    return {"workload": workload, "source_sha": source_sha(), "copy_mib": copy_mib,
            "fetch_scale": f_scale, "write_scale": w_scale, "kernels": kernels}


def mfma_table(path: str, simds: int = 1024, xcds: int = 8) -> str:
    """MFMA use per kernel from one counter run of SQ_VALU_MFMA_BUSY_CYCLES,
    GRBM_GUI_ACTIVE and SQ_INSTS_VALU_MFMA_MOPS_BF16 (medians over the
    dispatches). GRBM_GUI_ACTIVE comes summed over the XCDs, so the busy
    fraction is MFMA-busy SIMD cycles / (GPU-active cycles / XCDs x SIMDs,
    4 per CU); the MOPS counter counts 512 flops, and the achieved rate
    divides them by the dispatch's own start-to-end time in the counter run."""
    per = defaultdict(dict)
    for r in csv.DictReader(open(path)):
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        d = per[key]
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    by_kernel = defaultdict(list)
    for (name, _), d in per.items():
        k = short_name(name)
        if k is None or "GRBM_GUI_ACTIVE" not in d or d["GRBM_GUI_ACTIVE"] <= 0:
            continue
        busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (d["GRBM_GUI_ACTIVE"] / xcds * simds)
        flops = d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        by_kernel[k].append((busy, flops, flops / max(1, d["ns"]) / 1e3))
    out = ["| kernel | dispatches | MFMA busy (% of SIMD cycles) | bf16 MFMA GFLOP per dispatch | "
           "TFLOP/s in the counter run |", "|---|---|---|---|---|"]
    for k in sorted(by_kernel):
        v = by_kernel[k]
        med = lambda i: sorted(x[i] for x in v)[len(v) // 2]  # noqa: E731
        out.append(f"| `{k}` | {len(v)} | {100 * med(0):.1f} | {med(1) / 1e9:.2f} | {med(2):.0f} |")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=float, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.csv))
    elif a.cmd == "mfma":
        print(mfma_table(a.csv))
    else:
        res = traffic(a.fetch, a.write, a.copy_mib, a.workload)
        with open(a.out, "w") as f:
            json.dump(res, f, indent=1)
        print(json.dumps(res, indent=1))


if __name__ == "__main__":
    sys.exit(main())
