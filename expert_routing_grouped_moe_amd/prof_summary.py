"""Condenses rocprofv3 CSV output into the short markdown tables kept under profiles/.

  python -m expert_routing_grouped_moe_amd.prof_summary stats    <run_kernel_stats.csv>
  python -m expert_routing_grouped_moe_amd.prof_summary counters <run_counter_collection.csv>

`stats` lists every kernel of the trace (calls, average/min/max duration). `counters` averages
each hardware counter per dispatch, per kernel.
"""
from __future__ import annotations

import csv
import re
import sys
from collections import defaultdict


def short_name(name: str) -> str:
    n = re.sub(r"\(anonymous namespace\)::", "", name)
    n = re.sub(r"\(.*\)$", "", n)           # drop the parameter list
    n = n.replace("void ", "")
    return n[:90]


def stats_table(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.2f} |")
    return "\n".join(out)


def counters_table(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    acc = defaultdict(lambda: defaultdict(list))
    for r in rows:
        acc[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for k in acc.values() for c in k})
    out = ["| kernel | dispatches | " + " | ".join(f"{c} (avg/dispatch)" for c in names) + " |",
           "|---|---|" + "---|" * len(names)]
    for kern, cs in acc.items():
        n = max(len(v) for v in cs.values())
        vals = " | ".join(f"{sum(cs[c]) / len(cs[c]):.1f}" if cs.get(c) else "-" for c in names)
        out.append(f"| `{kern}` | {n} | {vals} |")
    return "\n".join(out)


if __name__ == "__main__":
    mode, path = sys.argv[1], sys.argv[2]
    print(stats_table(path) if mode == "stats" else counters_table(path))
