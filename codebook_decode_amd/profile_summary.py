"""Render a rocprofv3 kernel-stats CSV (--stats --output-format csv) as a short
markdown table (used to write the summaries under profiles/).

    python -m codebook_decode_amd.profile_summary <run_kernel_stats.csv> "<title>" "<command>" [notes...]
"""
from __future__ import annotations

import csv
import re
import sys


def short(name: str) -> str:
    name = re.sub(r"\(.*", "", name).replace("void ", "")
    return name


def render(path: str, title: str, command: str, notes: list) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"# {title}", "", "Command (repository root on the GPU box):", "", f"    {command}", ""]
    out += notes + [""] if notes else []
    out += ["| kernel | calls | total us | avg us | min us | max us | % |", "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        n = short(r["Name"])
        if not n.startswith("hr::"):
            continue
        out.append(f"| {n} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e3:.0f} | "
                   f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    print(render(sys.argv[1], sys.argv[2], sys.argv[3], sys.argv[4:]), end="")
