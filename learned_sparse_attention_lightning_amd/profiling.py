"""Summaries of rocprofv3 output for the DSA kernels.

    python -m learned_sparse_attention_lightning_amd.profiling trace DB OUT.md --command "..."
    python -m learned_sparse_attention_lightning_amd.profiling traffic \
        --kernel-fetch DIR --kernel-write DIR --copy-fetch DIR --copy-write DIR \
        --copy-bytes N --kernel REGEX --source FILE --out OUT.json --command "..."

    python -m learned_sparse_attention_lightning_amd.profiling counters \
        --run DIR [--run DIR ...] --kernel NAME=REGEX [...] --out OUT.md --command "..."

`trace` turns the kernel table of a `rocprofv3 --kernel-trace --stats` run
(the rocpd SQLite database) into a short markdown table.  `counters` turns
`rocprofv3 --pmc` runs (one per counter set) into per-dispatch averages per
kernel, with the matrix-core busy fractions they imply.  `traffic` turns two
`--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of a kernel into HBM bytes per
dispatch, each counter scaled by what it reads for a plain copy of a known
number of bytes (the copy reads and writes exactly that many bytes).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sqlite3


def kernel_table(db_path: str):
    con = sqlite3.connect(db_path)
    rows = con.execute("select name, total_calls, total_duration, average, percentage "
                       "from top_kernels").fetchall()
    con.close()
    return rows


def short_name(name: str) -> str:
    m = re.search(r"(\w+_kernel(<[^>]*>)?)", name)
    return m.group(1) if m else name[:60]


def write_trace(db_path: str, out_md: str, command: str, title: str):
    rows = kernel_table(db_path)
    lines = [f"# {title}", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | avg (us) | total (ms) | share |", "|---|---|---|---|---|"]
    for name, calls, total, avg, pct in rows:
        lines.append(f"| `{short_name(name)}` | {calls} | {avg:.2f} | {total / 1e3:.3f} | "
                     f"{pct:.1f}% |")
    lines.append("")
    lines.append("Durations are GPU execution times of each dispatch (rocprofv3 kernel trace); "
                 "kernels outside the library are torch's input generation.")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def counter_per_dispatch(run_dir: str, counter: str, kernel_regex: str) -> float:
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    vals = {}
    for fn in files:
        for r in csv.DictReader(open(fn)):
            if r["Counter_Name"] != counter or not re.search(kernel_regex, r["Kernel_Name"]):
                continue
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        raise ValueError(f"no {counter} samples for /{kernel_regex}/ under {run_dir}")
    return sum(vals.values()) / len(vals)


def counter_table(run_dirs, kernel_regex: str):
    """{counter: mean per dispatch} of the dispatches whose name matches."""
    out = {}
    for d in run_dirs:
        per = {}
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(fn)):
                if not re.search(kernel_regex, r["Kernel_Name"]):
                    continue
                key = (r["Counter_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        sums = {}
        for (c, _), v in per.items():
            sums.setdefault(c, []).append(v)
        for c, vs in sums.items():
            out[c] = (sum(vs) / len(vs), len(vs))
    return out


# SIMDs and XCDs of the device: the matrix-core busy cycles are summed over
# SIMDs, GRBM_GUI_ACTIVE over XCDs, SQ_BUSY_CU_CYCLES over SIMDs in
# quad-cycles.
DEVICE_SIMDS = 1024
DEVICE_XCDS = 8


def write_counters(a):
    kernels = [k.split("=", 1) for k in a.kernel]
    lines = [f"# {a.title}", "", "Commands (one rocprofv3 run per counter set):", "", "```"]
    lines += a.command
    lines += ["```", ""]
    for label, regex in kernels:
        tab = counter_table(a.run, regex)
        if not tab:
            raise ValueError(f"no samples for {label} (/{regex}/)")
        lines += [f"## `{label}`", "", "| counter | per dispatch | dispatches |", "|---|---|---|"]
        for c in sorted(tab):
            v, n = tab[c]
            lines.append(f"| {c} | {v:,.0f} | {n} |")
        derived = []
        mf = tab.get("SQ_VALU_MFMA_BUSY_CYCLES", (None,))[0]
        busy = tab.get("SQ_BUSY_CU_CYCLES", (None,))[0]
        grbm = tab.get("GRBM_GUI_ACTIVE", (None,))[0]
        co = tab.get("SQ_VALU_MFMA_COEXEC_CYCLES", (None,))[0]
        if mf is not None and busy:
            derived.append(f"matrix cores busy, share of SIMD-busy cycles: "
                           f"{mf / (4 * busy):.3f} (SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES))")
        if mf is not None and grbm:
            cyc = grbm / DEVICE_XCDS
            derived.append(f"matrix cores busy, share of the kernel's cycles: "
                           f"{mf / (DEVICE_SIMDS * cyc):.3f} (over {DEVICE_SIMDS} SIMDs x "
                           f"GRBM_GUI_ACTIVE / {DEVICE_XCDS} = {cyc:,.0f} cycles)")
        if mf and co is not None:
            derived.append(f"VALU issued while the matrix cores are busy: {co / mf:.3f} of their "
                           f"busy cycles (SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES)")
        if "FETCH_SIZE" in tab:
            derived.append(f"FETCH_SIZE: {tab['FETCH_SIZE'][0] / 1024:,.1f} MiB per dispatch "
                           f"(uncalibrated counter units of KiB)")
        if derived:
            lines += [""] + [f"- {d}" for d in derived]
        lines.append("")
    if a.note:
        lines += [a.note, ""]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def source_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def write_traffic(a):
    kf = counter_per_dispatch(a.kernel_fetch, "FETCH_SIZE", a.kernel)
    kw = counter_per_dispatch(a.kernel_write, "WRITE_SIZE", a.kernel)
    cf = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cw = counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    f_fetch = a.copy_bytes / cf
    f_write = a.copy_bytes / cw
    rec = {"kernel": a.kernel, "workload": a.workload,
           "source": os.path.basename(a.source), "source_sha256_16": source_hash(a.source),
           "fetch_counter_per_dispatch": kf, "write_counter_per_dispatch": kw,
           "copy_bytes": a.copy_bytes, "copy_fetch_counter": cf, "copy_write_counter": cw,
           "bytes_per_fetch_unit": f_fetch, "bytes_per_write_unit": f_write,
           "hbm_read_bytes_per_launch": kf * f_fetch, "hbm_write_bytes_per_launch": kw * f_write,
           "hbm_bytes_per_launch": kf * f_fetch + kw * f_write, "command": a.command}
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("out")
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="Kernel trace")
    tr = sub.add_parser("traffic")
    for k in ("kernel_fetch", "kernel_write", "copy_fetch", "copy_write"):
        tr.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    tr.add_argument("--copy-bytes", type=int, required=True)
    tr.add_argument("--copy-kernel", default="copy")
    tr.add_argument("--kernel", required=True)
    tr.add_argument("--workload", required=True)
    tr.add_argument("--source", required=True)
    tr.add_argument("--out", required=True)
    tr.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--run", action="append", required=True)
    c.add_argument("--kernel", action="append", required=True, help="LABEL=REGEX")
    c.add_argument("--out", required=True)
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--title", default="Counters")
    c.add_argument("--note", default="")
    a = ap.parse_args()
    if a.cmd == "trace":
        write_trace(a.db, a.out, a.command, a.title)
    elif a.cmd == "counters":
        write_counters(a)
    else:
        print(json.dumps(write_traffic(a), indent=1))


if __name__ == "__main__":
    main()
