"""Summaries of rocprofv3 CSV output for the sampling kernels.

    python -m token_sampling_scaled_amd.profiling trace  --stats K.csv --workload W --command CMD
    python -m token_sampling_scaled_amd.profiling traffic --fetch F.csv --write W.csv \
        --copy-mib 512 --kernel rows_fast_bf16 [more kernels] --workload W --algorithmic-bytes B \
        --command-fetch CMD1 --command-write CMD2

    python -m token_sampling_scaled_amd.profiling counters --csv A.csv B.csv \
        --kernel rows_topp_hist --workload W --command CMD1 CMD2

`trace` turns a `--kernel-trace --stats` kernel_stats.csv into a short text
table.  `counters` averages the counters of every `--pmc` pass given (one
counter_collection.csv each) over the dispatches of the kernels whose name
contains --kernel, one row per counter.  `traffic` turns two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` passes into
HBM bytes per launch of one kernel: each counter (KiB per dispatch) is scaled by
what the same counter reads for a plain device copy of known size run in the
same process, and the record carries a digest of the library's kernel sources,
so a reader (bench.py) can tell whether the kernel has changed since.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
RECORD_TAG = "traffic_record:"


def source_digest() -> str:
    """sha256 over every kernel source of the library (names and contents)."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if os.path.splitext(path)[1] not in (".hip", ".hpp", ".cpp", ".h"):
            continue
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_records(profiles_dir: str):
    """Every traffic record found in the text summaries under profiles_dir."""
    out = []
    for path in sorted(glob.glob(os.path.join(profiles_dir, "*"))):
        if not os.path.isfile(path):
            continue
        with open(path, encoding="utf-8", errors="replace") as f:
            for line in f:
                line = line.strip().strip("`")
                if line.startswith(RECORD_TAG):
                    out.append(json.loads(line[len(RECORD_TAG):]))
    return out


def per_dispatch(counter_csv: str):
    """{dispatch id: (kernel name, {counter: value summed over instances})}."""
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    with open(counter_csv, newline="") as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            vals[d][r["Counter_Name"]] += float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
    return {d: (names[d], dict(v)) for d, v in vals.items()}


def _kernel_mean(disp, match: str, counter: str):
    xs = [c[counter] for name, c in disp.values() if match in name and counter in c]
    if not xs:
        raise SystemExit(f"no dispatch of a kernel matching {match!r} with {counter}")
    names = sorted({name for name, c in disp.values() if match in name})
    return sum(xs) / len(xs), len(xs), names


def _copy_reading(disp, counter: str):
    """Largest reading of the plain copy kernel (the calibration copy)."""
    xs = [c[counter] for name, c in disp.values() if "copyBuffer" in name and counter in c]
    if not xs:
        raise SystemExit("no copy-kernel dispatch to calibrate against")
    return max(xs)


def cmd_trace(a):
    lines = [f"# kernel trace: {a.workload}", "", "Command (from the repository root):", "",
             "```", a.command, "```", "",
             "| kernel | calls | average us | min us | max us | share % |",
             "|---|---|---|---|---|---|"]
    with open(a.stats, newline="") as f:
        for r in csv.DictReader(f):
            lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.2f} |")
    print("\n".join(lines))


def cmd_traffic(a):
    """One launch of the path: the sum, over the kernels named by --kernel (one
    match string per kernel the call launches), of their mean per dispatch."""
    fd = per_dispatch(a.fetch)
    wd = per_dispatch(a.write)
    copy_kib = a.copy_mib * 1024.0
    f_copy = _copy_reading(fd, "FETCH_SIZE")
    w_copy = _copy_reading(wd, "WRITE_SIZE")
    f_scale = copy_kib / f_copy
    w_scale = copy_kib / w_copy
    rows = []
    fetch_b = write_b = 0.0
    names_all = []
    for match in a.kernel:
        f_mean, f_n, names = _kernel_mean(fd, match, "FETCH_SIZE")
        w_mean, w_n, _ = _kernel_mean(wd, match, "WRITE_SIZE")
        fetch_b += f_mean * f_scale * 1024.0
        write_b += w_mean * w_scale * 1024.0
        names_all.append(names[0])
        rows.append((names[0], f_mean, f_n, w_mean, w_n))
    rec = {"workload": a.workload, "kernel": " + ".join(names_all), "bytes_per_launch": fetch_b + write_b,
           "fetch_bytes": fetch_b, "write_bytes": write_b, "fetch_scale": f_scale,
           "write_scale": w_scale, "source_sha256": source_digest()}
    lines = [f"# HBM traffic: {a.workload}", "",
             "Two counter passes (from the repository root):", "",
             "```", a.command_fetch, a.command_write, "```", "",
             f"Calibration: a plain copy of {a.copy_mib} MiB reads FETCH_SIZE {f_copy:.1f} KiB "
             f"(scale {f_scale:.4f}) and WRITE_SIZE {w_copy:.1f} KiB (scale {w_scale:.4f}).", "",
             "| kernel | FETCH_SIZE KiB per dispatch (dispatches) | WRITE_SIZE KiB per dispatch | "
             "bytes per launch |", "|---|---|---|---|"]
    for name, f_mean, f_n, w_mean, w_n in rows:
        lines.append(f"| `{name}` | {f_mean:.1f} ({f_n}) | {w_mean:.1f} ({w_n}) | "
                     f"{(f_mean * f_scale + w_mean * w_scale) * 1024.0:,.0f} |")
    lines.append("")
    lines.append(f"Per launch of the call: fetch {fetch_b:,.0f} B, write {write_b:,.0f} B.")
    if a.algorithmic_bytes:
        lines.append(f"Algorithmic bytes per launch: {a.algorithmic_bytes:,}; measured / "
                     f"algorithmic = {(fetch_b + write_b) / a.algorithmic_bytes:.4f}.")
    lines.append("")
    lines.append("`" + RECORD_TAG + " " + json.dumps(rec) + "`")
    print("\n".join(lines))


def cmd_counters(a):
    per = collections.defaultdict(list)
    names = set()
    for path in a.csv:
        for name, c in per_dispatch(path).values():
            if a.kernel not in name:
                continue
            names.add(name)
            for k, v in c.items():
                per[k].append(v)
    if not per:
        raise SystemExit(f"no dispatch of a kernel matching {a.kernel!r}")
    lines = [f"# counters: {a.kernel} on {a.workload}", "", "Counter passes (from the repository root):",
             "", "```", *a.command, "```", "", "Kernels: " + ", ".join(f"`{n}`" for n in sorted(names)),
             "", "| counter | mean per dispatch | dispatches |", "|---|---|---|"]
    for k in sorted(per):
        xs = per[k]
        lines.append(f"| {k} | {sum(xs) / len(xs):,.0f} | {len(xs)} |")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--stats", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True)
    p = sub.add_parser("traffic")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--copy-mib", type=int, required=True)
    p.add_argument("--kernel", nargs="+", required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--algorithmic-bytes", type=int, default=0)
    p.add_argument("--command-fetch", required=True)
    p.add_argument("--command-write", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--csv", nargs="+", required=True)
    c.add_argument("--kernel", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--command", nargs="+", required=True)
    a = ap.parse_args(argv)
    {"trace": cmd_trace, "traffic": cmd_traffic, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
