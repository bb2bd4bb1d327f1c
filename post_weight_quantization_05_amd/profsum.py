"""Summarize rocprofv3 CSV output (kernel stats and counter collections) for the profile notes.

python -m post_weight_quantization_05_amd.profsum stats <dir>          per-kernel time table
python -m post_weight_quantization_05_amd.profsum counters <dir> [substr]  per-dispatch counter sums
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


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    else:
        print(counters(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""))
