"""HBM traffic of the library's kernels from rocprofv3 counter runs, and its check against the sources.

Two ``rocprofv3 --pmc`` runs of ``bench.py --copy-probe`` (one with FETCH_SIZE, one with WRITE_SIZE) give the
kilobytes each dispatch moved between L2 and memory.  The probe copy of a known size in the same runs
calibrates both counters: traffic = counter x (known copy bytes / what the counter read for the copy).  The
summary written here records, per kernel, the calibrated bytes per launch and a hash of the sources the kernel
is built from; ``bench.py`` reports the figure only while that hash still matches the sources.

    python -m hierarchical_sparse_attention_mean_amd.profiling traffic --fetch DIR --write DIR \
        --copy-bytes N --kernel NAME --workload NAME --command "..." > profiles/NAME_WORKLOAD_traffic.md

The ``kernel-stats`` subcommand turns a ``rocprofv3 --kernel-trace --stats`` run into the per-kernel table kept
under ``profiles/``.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")

# sources each kernel is compiled from (its translation unit and the headers it includes)
_COMMON = ["common.hpp", "entries.hpp", "persist.hpp", "launch.hpp"]
KERNEL_SOURCES = {
    "attn_fwd_bf16": ["attn_fwd.hip"] + _COMMON,
    "bwd_dq_bf16": ["attn_bwd.hip"] + _COMMON,
    "bwd_dkdv_bf16": ["attn_bwd.hip"] + _COMMON,
    "coarse_reduce": ["attn_bwd.hip"] + _COMMON,
    "pool_levels12": ["pyramid.hip", "common.hpp", "launch.hpp"],
    "select_level": ["select.hip", "common.hpp", "launch.hpp"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, summed counter value)} from a rocprofv3 counter_collection CSV."""
    out = {}
    acc = collections.defaultdict(float)
    names = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = r["Dispatch_Id"]
            acc[d] += float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
    for d, v in acc.items():
        out[d] = (names[d], v)
    return out


def _csv_in(directory: str) -> str:
    hits = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    return hits[0]


def _kernel_and_copy(rows, kernel: str):
    mine = [v for (nm, v) in rows.values() if re.search(r"\b" + kernel + r"\b", nm)]
    copies = [v for (nm, v) in rows.values() if re.search(r"copy", nm, re.I)]
    if not mine or not copies:
        raise ValueError(f"need dispatches of {kernel} and of the probe copy")
    return sum(mine) / len(mine), len(mine), max(copies)


def traffic_summary(fetch_dir: str, write_dir: str, copy_bytes: int, kernel: str, workload: str,
                    command: str) -> str:
    fk, nf, fc = _kernel_and_copy(_per_dispatch(_csv_in(fetch_dir), "FETCH_SIZE"), kernel)
    wk, nw, wc = _kernel_and_copy(_per_dispatch(_csv_in(write_dir), "WRITE_SIZE"), kernel)
    ff = copy_bytes / (fc * 1024.0)
    fw = copy_bytes / (wc * 1024.0)
    fetch_b = fk * 1024.0 * ff
    write_b = wk * 1024.0 * fw
    lines = [
        f"# HBM traffic of {kernel} on the {workload} workload",
        "",
        "Commands (from the repository root, on one MI355X):",
        "",
        "```",
        command,
        "```",
        "",
        "| quantity | FETCH_SIZE | WRITE_SIZE |",
        "|---|---|---|",
        f"| {kernel}: KiB per dispatch (mean of {nf} / {nw} dispatches) | {fk:.0f} | {wk:.0f} |",
        f"| probe copy of {copy_bytes} bytes: KiB read by the counter | {fc:.0f} | {wc:.0f} |",
        f"| calibration factor (known bytes / counter bytes) | {ff:.4f} | {fw:.4f} |",
        f"| {kernel}: calibrated bytes per launch | {fetch_b:.4g} | {write_b:.4g} |",
        "",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.6g}",
        f"source_sha256: {source_hash(kernel)}",
        "",
    ]
    return "\n".join(lines)


def read_traffic(kernel: str, workload: str):
    """Calibrated bytes per launch from the committed summary, or None if absent or the sources changed."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    text = open(path).read()
    m = re.search(r"^traffic_bytes_per_launch: (\S+)$", text, re.M)
    h = re.search(r"^source_sha256: (\S+)$", text, re.M)
    if not m or not h or h.group(1) != source_hash(kernel):
        return None
    return float(m.group(1))


def kernel_stats_summary(directory: str, title: str, command: str) -> str:
    """Markdown table of a rocprofv3 --kernel-trace --stats run (its kernel_stats.csv)."""
    hits = glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no kernel_stats.csv under {directory}")
    lines = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "```", command, "```", "",
             "Source: the run's kernel_stats.csv (kernel trace, every launch including the warm-up steps).", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    with open(hits[0]) as f:
        for r in csv.DictReader(f):
            m = re.search(r"::(\w+)(<[^>]*>)?\(", r["Name"])
            short = (m.group(1) + (m.group(2) or "")) if m else r["Name"][:40]
            lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                         f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    lines.append("")
    return "\n".join(lines)


def l2_hits_summary(directory: str, kernels: list, title: str, command: str) -> str:
    """L2 (TCC) hit rate per kernel from a rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum run: mean per dispatch."""
    path = _csv_in(directory)
    hit, miss = _per_dispatch(path, "TCC_HIT_sum"), _per_dispatch(path, "TCC_MISS_sum")
    lines = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "```", command, "```", "",
             "| kernel | dispatches | L2 hits per dispatch | L2 misses per dispatch | hit rate |", "|---|---|---|---|---|"]
    for k in kernels:
        ds = [d for d, (nm, _) in hit.items() if k in nm and d in miss]
        if not ds:
            continue
        h = sum(hit[d][1] for d in ds) / len(ds)
        m = sum(miss[d][1] for d in ds) / len(ds)
        lines.append(f"| {k} | {len(ds)} | {h:.4g} | {m:.4g} | {h / max(h + m, 1.0):.3f} |")
    lines.append("")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    ks = sub.add_parser("kernel-stats")
    ks.add_argument("--dir", required=True)
    ks.add_argument("--title", required=True)
    ks.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True)
    h = sub.add_parser("l2-hits")
    h.add_argument("--dir", required=True)
    h.add_argument("--kernels", required=True, help="comma-separated kernel name substrings")
    h.add_argument("--title", required=True)
    h.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.cmd == "kernel-stats":
        print(kernel_stats_summary(a.dir, a.title, a.command))
    elif a.cmd == "l2-hits":
        print(l2_hits_summary(a.dir, a.kernels.split(","), a.title, a.command))
    else:
        print(traffic_summary(a.fetch, a.write, a.copy_bytes, a.kernel, a.workload, a.command))


if __name__ == "__main__":
    main()
