"""HBM traffic of the library's kernels from rocprofv3 counter runs, and its check against the sources.

Two ``rocprofv3 --pmc`` runs of ``bench.py --copy-probe`` (one with FETCH_SIZE, one with WRITE_SIZE) give the
kilobytes each dispatch moved between L2 and memory.  The probe copy of a known size in the same runs
calibrates both counters: traffic = counter x (known copy bytes / what the counter read for the copy).  The
summary written here records, per kernel, the calibrated bytes per launch and a hash of the sources the kernel
is built from; ``bench.py`` reports the figure only while that hash still matches the sources.

    python -m hierarchical_sparse_attention_mean_amd.profiling traffic --fetch DIR --write DIR \
        --copy-bytes N --kernel NAME --workload NAME --command "..." > profiles/NAME_WORKLOAD_traffic.md

The ``kernel-stats`` subcommand turns a ``rocprofv3 --kernel-trace --stats`` run into the per-kernel table kept
under ``profiles/``; ``counters`` turns ``rocprofv3 --pmc`` runs of other counters (MFMA busy cycles, LDS bank
conflicts, texture-unit busy, wave wait cycles) into per-kernel means and derived percentages.
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
    "attn_fwd_pair_bf16": ["attn_fwd.hip"] + _COMMON,
    "bwd_dq_bf16": ["attn_bwd.hip"] + _COMMON,
    "bwd_dkdv_bf16": ["attn_bwd.hip"] + _COMMON,
    "reduce_and_order": ["attn_bwd.hip"] + _COMMON,
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


CUS, SIMDS, XCDS = 256, 1024, 8   # MI355X: compute units, SIMDs (4 per CU), XCDs


def _per_dispatch_all(path: str):
    """{dispatch id: (kernel name, {counter: value})} from a counter_collection CSV, each counter summed over the
    rows it has for the dispatch.  GRBM_GUI_ACTIVE comes as one row holding the sum over the XCDs (it reads about
    8x the dispatch's duration in cycles), so the kernel's cycles are GRBM_GUI_ACTIVE / 8; the summary checks this
    against the dispatch's timestamps (the implied clock).  The dispatch duration (ns) is kept as 'duration_ns'."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    names, dur = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = r["Dispatch_Id"]
            vals[d][r["Counter_Name"]].append(float(r["Counter_Value"]))
            names[d] = r["Kernel_Name"]
            dur[d] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    out = {}
    for d, cs in vals.items():
        c = {k: sum(v) for k, v in cs.items()}
        if "GRBM_GUI_ACTIVE" in c:
            c["GRBM_GUI_ACTIVE"] /= XCDS
        c["duration_ns"] = dur[d]
        out[d] = (names[d], c)
    return out


# derived figures: (label, counters needed, formula over the per-dispatch means)
_DERIVED = [
    ("dispatch duration, us (timestamps)", ("duration_ns",), lambda c: c["duration_ns"] / 1e3),
    ("implied clock, GHz (GRBM_GUI_ACTIVE / 8 / duration)", ("GRBM_GUI_ACTIVE", "duration_ns"),
     lambda c: c["GRBM_GUI_ACTIVE"] / c["duration_ns"]),
    ("MFMA busy, % of SIMD cycles", ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"),
     lambda c: 100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] * SIMDS)),
    ("bf16 MFMA TFLOP issued per dispatch", ("SQ_INSTS_VALU_MFMA_MOPS_BF16",),
     lambda c: c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e12),
    ("LDS bank conflicts, % of LDS active cycles", ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"),
     lambda c: 100.0 * c["SQ_LDS_BANK_CONFLICT"] / max(c["SQ_LDS_IDX_ACTIVE"], 1.0)),
    ("LDS active, % of CU cycles", ("SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"),
     lambda c: 100.0 * c["SQ_LDS_IDX_ACTIVE"] / (c["GRBM_GUI_ACTIVE"] * CUS)),
    ("texture address (TA) busy, % of CU cycles", ("TA_TA_BUSY_sum", "GRBM_GUI_ACTIVE"),
     lambda c: 100.0 * c["TA_TA_BUSY_sum"] / (c["GRBM_GUI_ACTIVE"] * CUS)),
    ("texture data (TD) busy, % of CU cycles", ("TD_TD_BUSY_sum", "GRBM_GUI_ACTIVE"),
     lambda c: 100.0 * c["TD_TD_BUSY_sum"] / (c["GRBM_GUI_ACTIVE"] * CUS)),
    ("CU busy, % of cycles", ("SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"),
     lambda c: 100.0 * c["SQ_BUSY_CU_CYCLES"] / (c["GRBM_GUI_ACTIVE"] * CUS)),
    ("VALU instructions issued, % of wave cycles", ("SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"),
     lambda c: 100.0 * c["SQ_ACTIVE_INST_VALU"] / max(c["SQ_WAVE_CYCLES"], 1.0)),
    ("LDS instructions issued, % of wave cycles", ("SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES"),
     lambda c: 100.0 * c["SQ_ACTIVE_INST_LDS"] / max(c["SQ_WAVE_CYCLES"], 1.0)),
    ("vector memory instructions issued, % of wave cycles", ("SQ_ACTIVE_INST_VMEM", "SQ_WAVE_CYCLES"),
     lambda c: 100.0 * c["SQ_ACTIVE_INST_VMEM"] / max(c["SQ_WAVE_CYCLES"], 1.0)),
    ("waves waiting on a dependency (s_waitcnt), % of wave cycles", ("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
     lambda c: 100.0 * c["SQ_WAIT_INST_ANY"] / max(c["SQ_WAVE_CYCLES"], 1.0)),
    ("waves waiting for anything, % of wave cycles", ("SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
     lambda c: 100.0 * c["SQ_WAIT_ANY"] / max(c["SQ_WAVE_CYCLES"], 1.0)),
    # SQ_WAVE_CYCLES counts in units of 4 cycles: waves per SIMD = 4 SQ_WAVE_CYCLES / (cycles * SIMDS)
    ("resident waves per SIMD (average)", ("SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"),
     lambda c: 4.0 * c["SQ_WAVE_CYCLES"] / (c["GRBM_GUI_ACTIVE"] * SIMDS)),
]


def counters_summary(directories: list, kernels: list, title: str, commands: list) -> str:
    """Per-kernel means of raw counters over the dispatches of one or more rocprofv3 --pmc runs, and the derived
    figures that the counters present allow (MFMA busy, LDS bank conflicts, TA/TD busy, where waves wait)."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in directories:
        for _, (nm, cs) in _per_dispatch_all(_csv_in(d)).items():
            for k in kernels:
                if re.search(r"\b" + k + r"\b", nm):
                    for c, v in cs.items():
                        per[k][c].append(v)
    lines = [f"# {title}", "", "Commands (from the repository root, on one MI355X):", "", "```", *commands, "```", "",
             "Counters are summed over their hardware instances per dispatch, then averaged over the dispatches; kernel "
             f"cycles = GRBM_GUI_ACTIVE / {XCDS} (the counter sums the XCDs); {CUS} CUs, {SIMDS} SIMDs.  Profiled "
             "dispatches run one at a time (the transpose is not beside the forward).", ""]
    for k in kernels:
        if k not in per:
            continue
        mean = {c: sum(v) / len(v) for c, v in per[k].items()}
        nd = max(len(v) for v in per[k].values())
        lines += [f"## {k}", "", f"dispatches: {nd}", "", "| derived | value |", "|---|---|"]
        for label, need, f in _DERIVED:
            if all(n in mean for n in need):
                lines.append(f"| {label} | {f(mean):.4g} |")
        lines += ["", "| counter | mean per dispatch |", "|---|---|"]
        for c in sorted(mean):
            lines.append(f"| {c} | {mean[c]:.6g} |")
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
    cs = sub.add_parser("counters")
    cs.add_argument("--dirs", required=True, help="comma-separated rocprofv3 --pmc output directories")
    cs.add_argument("--kernels", required=True, help="comma-separated kernel names")
    cs.add_argument("--title", required=True)
    cs.add_argument("--command", action="append", required=True)
    a = ap.parse_args()
    if a.cmd == "counters":
        print(counters_summary(a.dirs.split(","), a.kernels.split(","), a.title, a.command))
        return
    if a.cmd == "kernel-stats":
        print(kernel_stats_summary(a.dir, a.title, a.command))
    elif a.cmd == "l2-hits":
        print(l2_hits_summary(a.dir, a.kernels.split(","), a.title, a.command))
    else:
        print(traffic_summary(a.fetch, a.write, a.copy_bytes, a.kernel, a.workload, a.command))


if __name__ == "__main__":
    main()
