"""Render rocprofv3 CSV output as the short markdown summaries under profiles/.

    python -m codebook_decode_amd.profile_summary <run_kernel_stats.csv> "<title>" "<command>" [notes...]
    python -m codebook_decode_amd.profile_summary traffic <fetch counter_collection.csv> \
        <write counter_collection.csv> "<fetch command>" "<write command>"

The traffic form reads FETCH_SIZE and WRITE_SIZE (KiB per dispatch) for the
gate/up GEMM and for a plain 256 MiB device copy, scales the GEMM's readings by
the copy's (counter bytes / bytes the copy must move) and records the
SHA-256 of the GEMM source the counters were taken on.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import os
import re
import sys


def short(name: str) -> str:
    name = re.sub(r"\(.*", "", name).replace("void ", "")
    return name


def render(path: str, title: str, command: str, notes: list) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"# {title}", "", "Command (repository root on the MI355X host):", "", f"    {command}", ""]
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


COPY_BYTES = 256 << 20
GEMM_SOURCE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "gemm.hip")


def source_digest(path: str = GEMM_SOURCE) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def per_dispatch(path: str, counter: str) -> dict:
    """{kernel short name: [KiB per dispatch, ...]} for one counter."""
    acc = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        acc[key] += float(r["Counter_Value"])
        names[key] = short(r["Kernel_Name"])
    out = collections.defaultdict(list)
    for key, v in acc.items():
        out[names[key]].append(v)
    return out


def render_traffic(fetch_csv: str, write_csv: str, fetch_cmd: str, write_cmd: str) -> str:
    f, w = per_dispatch(fetch_csv, "FETCH_SIZE"), per_dispatch(write_csv, "WRITE_SIZE")
    gemm = [k for k in f if "gemm_tiled_kernel<2" in k][0]
    copy = [k for k in f if "copyBuffer" in k][0]                 # the 256 MiB device copy
    mean = lambda xs: sum(xs) / len(xs)
    f_gemm, w_gemm = mean(f[gemm]) * 1024, mean(w[gemm]) * 1024
    f_copy, w_copy = mean(f[copy]) * 1024, mean(w[copy]) * 1024
    kf, kw = f_copy / COPY_BYTES, w_copy / COPY_BYTES
    traffic = f_gemm / kf + w_gemm / kw
    algo = 19456 * 2560 * 2 + 512 * 2560 * 2 + 512 * 9728 * 2
    lines = [
        "# HBM traffic of the gate/up GEMM, M = 512 (512 x 19456 x 2560, bf16, SwiGLU epilogue)", "",
        "Commands (repository root on the MI355X host; one counter set per run):", "",
        f"    {fetch_cmd}", f"    {write_cmd}", "",
        "`codebook_decode_amd.traffic_probe` launches the GEMM on 3 distinct weight matrices, then a plain "
        "256 MiB device copy twice. The copy's readings against the 256 MiB it must read and write give the "
        "scale of each counter.", "",
        "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---:|---:|---:|",
        f"| {gemm} | {len(f[gemm])} | {f_gemm / 1024:.0f} | {w_gemm / 1024:.0f} |",
        f"| {copy} | {len(f[copy])} | {f_copy / 1024:.0f} | {w_copy / 1024:.0f} |", "",
        f"counter scale (copy): fetch {kf:.4f}, write {kw:.4f} of the bytes moved", "",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        f"algorithmic_bytes_per_launch: {algo}",
        f"traffic_over_algorithmic: {traffic / algo:.3f}",
        f"gemm_source_sha256: {source_digest()}", ""]
    return "\n".join(lines)


if __name__ == "__main__":
    if sys.argv[1] == "traffic":
        print(render_traffic(*sys.argv[2:6]), end="")
    else:
        print(render(sys.argv[1], sys.argv[2], sys.argv[3], sys.argv[4:]), end="")
