"""Summarize rocprofv3 CSV output (kernel stats and counter collections) for the profile notes.

python -m post_weight_quantization_05_amd.profsum stats <dir>          per-kernel time table
python -m post_weight_quantization_05_amd.profsum counters <dir> [substr]  per-dispatch counter sums
python -m post_weight_quantization_05_amd.profsum bykernel <dir> [from]   per-kernel counter means
python -m post_weight_quantization_05_amd.profsum durations <dir> [from]  per-kernel mean durations (trace)
python -m post_weight_quantization_05_amd.profsum clock <dir>             per-kernel clock and MFMA busy share
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


def clock(d: str, xcds: int = 8, simds: int = 1024) -> str:
    """Mean clock and MFMA-busy share per kernel, from a run with GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES.

    The collection CSV holds GRBM_GUI_ACTIVE summed over the XCDs, so one XCD's active cycles are the value
    over xcds; over the dispatch's duration that is the mean clock. The busy share is the MFMA-busy cycles
    summed over SIMDs over (active cycles x SIMDs). Short dispatches read high: the counters also see a few
    microseconds around the dispatch.
    """
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
    gui, busy, dur, kern = {}, {}, {}, {}
    for r in csv.DictReader(open(f)):
        disp = int(r["Dispatch_Id"])
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            gui[disp] = gui.get(disp, 0.0) + float(r["Counter_Value"])
        elif r["Counter_Name"] == "SQ_VALU_MFMA_BUSY_CYCLES":
            busy[disp] = busy.get(disp, 0.0) + float(r["Counter_Value"])
        dur[disp] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9
        kern[disp] = _short(r["Kernel_Name"])
    agg = collections.defaultdict(lambda: [0, 0.0, 0.0, 0.0])
    for disp, g in gui.items():
        a = agg[kern[disp]]
        a[0] += 1
        a[1] += g / xcds
        a[2] += dur[disp]
        a[3] += busy.get(disp, 0.0)
    out = ["| kernel | dispatches | total ms | mean clock GHz | MFMA busy % |", "|---|---|---|---|---|"]
    for k, (n, cyc, t, b) in sorted(agg.items(), key=lambda kv: -kv[1][2]):
        if t <= 0 or cyc <= 0:
            continue
        out.append(f"| `{k}` | {n} | {t * 1e3:.3f} | {cyc / t / 1e9:.3f} | {100 * b / (cyc * simds):.1f} |")
    return "\n".join(out)


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    elif sys.argv[1] == "bykernel":
        print(bykernel(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""))
    elif sys.argv[1] == "clock":
        print(clock(sys.argv[2]))
    elif sys.argv[1] == "durations":
        print(durations(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""))
    else:
        print(counters(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""))
