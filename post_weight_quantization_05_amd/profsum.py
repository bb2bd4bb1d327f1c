"""Summarize rocprofv3 CSV output (kernel stats and counter collections) for the profile notes.

python -m post_weight_quantization_05_amd.profsum stats <dir>          per-kernel time table
python -m post_weight_quantization_05_amd.profsum counters <dir> [substr]  per-dispatch counter sums
python -m post_weight_quantization_05_amd.profsum bykernel <dir> [from]   per-kernel counter means
python -m post_weight_quantization_05_amd.profsum durations <dir> [from]  per-kernel mean durations (trace)
  [from]: only the dispatches from the first one whose kernel name contains this text (a stage's kernels)
"""
from __future__ import annotations

import collections
import csv
import glob
import os
import sys


def _short(name: str) -> str:
    return name.replace("gptq::(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def stats(d: str) -> str:
    f = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(f)))
    out = ["| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out)


def counters(d: str, substr: str = "") -> str:
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
    agg = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(f)):
        if substr and substr not in r["Kernel_Name"]:
            continue
        key = (int(r["Dispatch_Id"]), r["Counter_Name"])
        agg[key] += float(r["Counter_Value"])
        names[int(r["Dispatch_Id"])] = _short(r["Kernel_Name"])
    out = ["| dispatch | kernel | counter | value |", "|---|---|---|---|"]
    for (disp, cn), v in sorted(agg.items()):
        out.append(f"| {disp} | `{names[disp]}` | {cn} | {v:.6g} |")
    return "\n".join(out)


def _first_dispatch(rows, start: str) -> int:
    ids = [int(r["Dispatch_Id"]) for r in rows if start and start in r["Kernel_Name"]]
    return min(ids) if ids else 0


def bykernel(d: str, start: str = "") -> str:
    """Mean over a kernel's dispatches of each counter (each dispatch's value summed over its instances)."""
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(f)))
    first = _first_dispatch(rows, start)
    per = collections.defaultdict(float)
    kern, dur = {}, {}
    for r in rows:
        if int(r["Dispatch_Id"]) < first:
            continue
        per[(int(r["Dispatch_Id"]), r["Counter_Name"])] += float(r["Counter_Value"])
        kern[int(r["Dispatch_Id"])] = _short(r["Kernel_Name"])
        dur[int(r["Dispatch_Id"])] = max(1, int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    agg = collections.defaultdict(list)
    for (disp, cn), v in per.items():
        agg[(kern[disp], cn)].append((v, dur[disp]))
    # the duration-weighted mean suits ratio counters (utilisations); durations are those of the profiled run
    out = ["| kernel | counter | dispatches | mean per dispatch | duration-weighted mean | total |",
           "|---|---|---|---|---|---|"]
    for (k, cn), vs in sorted(agg.items()):
        tot = sum(v for v, _ in vs)
        wmean = sum(v * t for v, t in vs) / sum(t for _, t in vs)
        out.append(f"| `{k}` | {cn} | {len(vs)} | {tot / len(vs):.6g} | {wmean:.6g} | {tot:.6g} |")
    return "\n".join(out)


def durations(d: str, start: str = "") -> str:
    """Mean and total duration per kernel from a kernel trace."""
    f = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)[0]
    rows = list(csv.DictReader(open(f)))
    first = _first_dispatch(rows, start)
    agg = collections.defaultdict(list)
    for r in rows:
        if int(r["Dispatch_Id"]) < first:
            continue
        agg[_short(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| kernel | dispatches | mean us | total us |", "|---|---|---|---|"]
    for k, vs in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| `{k}` | {len(vs)} | {sum(vs) / len(vs):.2f} | {sum(vs):.1f} |")
    return "\n".join(out)


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    elif sys.argv[1] == "bykernel":
        print(bykernel(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""))
    elif sys.argv[1] == "durations":
        print(durations(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""))
    else:
        print(counters(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""))
