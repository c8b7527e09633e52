"""Summaries of rocprofv3 output for the files under profiles/.

Two commands (run from the repository root on the CSV output of rocprofv3):

  python -m sparse_mla_attention_index_amd.rocprof_summary stats \\
      --stats <run dir>/run_kernel_stats.csv --out profiles/<name>.md --command "<cmd>"

writes a kernel-time table (calls, average / min / max ms, share of the total);

  python -m sparse_mla_attention_index_amd.rocprof_summary traffic \\
      --fetch <FETCH_SIZE run>/run_counter_collection.csv \\
      --write <WRITE_SIZE run>/run_counter_collection.csv \\
      --kernel idx_score --source sparse_mla_attention_index_amd/csrc/idx_score.hip \\
      --copy-bytes N --workload prefill-L65536-k2048 --out profiles/traffic_<workload>.json

averages FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the named kernel,
scales each by bytes / counter of the plain copy kernel of N bytes that the
same run executed (the runtime's device copy kernel, __amd_rocclr_copyBuffer,
which a same-dtype torch copy_ between device tensors launches), and records
the result with the
SHA-256 of the kernel's source file, so that a reader can tell whether the
kernel changed since the counters were taken;

  python -m sparse_mla_attention_index_amd.rocprof_summary table \\
      --fetch ... --write ... --kernel idx_score --kernel topk --kernel sparse_mla \\
      --copy-bytes N --out profiles/<name>.md --title "..." --command "<cmd>" ...

writes the same scaled figures for several kernels as a Markdown table;

  python -m sparse_mla_attention_index_amd.rocprof_summary counters \\
      --pmc <run 1>/run_counter_collection.csv --pmc <run 2>/... \\
      --stats <trace>/run_kernel_stats.csv --kernel idx_score ... --out profiles/<name>.md

derives per kernel from SQ/GRBM counters (averaged per dispatch) and the
trace's average duration: the shader clock (GRBM_GUI_ACTIVE summed over the
8 XCDs / 8 / duration), the matrix-core busy fraction
(SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x clock cycles)), and the share of wave
time spent waiting (SQ_WAIT_ANY, SQ_WAIT_INST_ANY; SQ_WAVE_CYCLES counts in
units of 4 cycles like them).
"""
import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict


def _per_dispatch(path, counter):
    """{dispatch_id: (kernel_name, value)} for one counter of a counter-collection CSV."""
    out = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = r["Dispatch_Id"]
            name, val = out.get(d, (r["Kernel_Name"], 0.0))
            out[d] = (name, val + float(r["Counter_Value"]))
    return out


def _kernel_avg(disp, substr):
    vals = [v for (name, v) in disp.values() if substr in name]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {substr!r}")
    return sum(vals) / len(vals), len(vals)


def _copy_counter(disp):
    """Counter value of the largest dispatch of the runtime's device-to-device
    copy kernel (the calibration copy; torch's dtype-conversion kernels also
    carry "copy" in their names and are not it)."""
    vals = [v for (name, v) in disp.values() if "copybuffer" in name.lower()]
    if not vals:
        raise SystemExit("no device copy kernel (copyBuffer) in the counter file")
    return max(vals)


def cmd_traffic(a):
    fetch = _per_dispatch(a.fetch, "FETCH_SIZE")
    write = _per_dispatch(a.write, "WRITE_SIZE")
    f_kib, nf = _kernel_avg(fetch, a.kernel)
    w_kib, nw = _kernel_avg(write, a.kernel)
    f_copy, w_copy = _copy_counter(fetch), _copy_counter(write)
    f_factor = a.copy_bytes / (f_copy * 1024.0)
    w_factor = a.copy_bytes / (w_copy * 1024.0)
    with open(a.source, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    rec = {
        "workload": a.workload,
        "kernel": a.kernel,
        "source": a.source,
        "source_sha256": sha,
        "dispatches": {"fetch_run": nf, "write_run": nw},
        "fetch_kib_per_dispatch": f_kib,
        "write_kib_per_dispatch": w_kib,
        "copy_bytes": a.copy_bytes,
        "copy_fetch_kib": f_copy,
        "copy_write_kib": w_copy,
        "fetch_factor": f_factor,
        "write_factor": w_factor,
        "traffic_bytes_per_launch": f_kib * 1024.0 * f_factor + w_kib * 1024.0 * w_factor,
        "commands": a.command,
    }
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def cmd_table(a):
    fetch = _per_dispatch(a.fetch, "FETCH_SIZE")
    write = _per_dispatch(a.write, "WRITE_SIZE")
    f_copy, w_copy = _copy_counter(fetch), _copy_counter(write)
    f_factor = a.copy_bytes / (f_copy * 1024.0)
    w_factor = a.copy_bytes / (w_copy * 1024.0)
    lines = [f"# {a.title}", "", "Commands (from the repository root, on the GPU host), one counter per run:", "",
             "```"] + list(a.command) + ["```", "",
             f"Calibration: the same runs copy {a.copy_bytes} bytes with a plain device copy, which reads "
             f"{f_copy:.0f} KiB by FETCH_SIZE and writes {w_copy:.0f} KiB by WRITE_SIZE, so FETCH_SIZE is "
             f"scaled by {f_factor:.4f} and WRITE_SIZE by {w_factor:.4f}.", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB (scaled) | written GB (scaled) |",
             "|---|---|---|---|---|---|"]
    for k in a.kernel:
        f_kib, nf = _kernel_avg(fetch, k)
        w_kib, _ = _kernel_avg(write, k)
        name = next(n for (n, _) in fetch.values() if k in n).replace("(anonymous namespace)::", "").split("(")[0]
        lines.append(f"| `{name}` | {nf} | {f_kib:.0f} | {w_kib:.0f} | {f_kib * 1024 * f_factor / 1e9:.2f} | "
                     f"{w_kib * 1024 * w_factor / 1e9:.2f} |")
    if a.note:
        lines += ["", a.note]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_counters(a):
    vals = defaultdict(dict)
    for path in a.pmc:
        with open(path, newline="") as f:
            rows = list(csv.DictReader(f))
        for k in a.kernel:
            acc, disp = defaultdict(float), set()
            for r in rows:
                if k in r["Kernel_Name"]:
                    acc[r["Counter_Name"]] += float(r["Counter_Value"])
                    disp.add(r["Dispatch_Id"])
            for c, v in acc.items():
                vals[k][c] = v / max(len(disp), 1)
    dur = {}
    with open(a.stats, newline="") as f:
        for r in csv.DictReader(f):
            for k in a.kernel:
                if k in r["Name"]:
                    dur[k] = float(r["AverageNs"]) * 1e-9
    lines = [f"# {a.title}", "", "Commands (from the repository root, on the GPU host):", "", "```"]
    lines += list(a.command) + ["```", ""]
    lines += ["| kernel | avg ms | clock GHz | MFMA busy | MFMA insts | VALU insts | LDS insts | wait (waitcnt/barrier) | wait (dependency) |",
              "|---|---|---|---|---|---|---|---|---|"]
    for k in a.kernel:
        v, t = vals[k], dur.get(k)
        if not t or "GRBM_GUI_ACTIVE" not in v:
            continue
        cyc = v["GRBM_GUI_ACTIVE"] / a.xcds
        ghz = cyc / t / 1e9
        busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (a.simds * cyc)
        wave = v.get("SQ_WAVE_CYCLES", 0.0) or 1.0
        name = next((r for r in [k]), k)
        lines.append(f"| `{name}` | {t * 1e3:.2f} | {ghz:.2f} | {100 * busy:.0f}% | {v.get('SQ_INSTS_MFMA', 0):.3g} | "
                     f"{v.get('SQ_INSTS_VALU', 0):.3g} | {v.get('SQ_INSTS_LDS', 0):.3g} | "
                     f"{100 * v.get('SQ_WAIT_ANY', 0) / wave:.0f}% | {100 * v.get('SQ_WAIT_INST_ANY', 0) / wave:.0f}% |")
    if a.note:
        lines += ["", a.note]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_stats(a):
    rows = []
    with open(a.stats, newline="") as f:
        for r in csv.DictReader(f):
            rows.append(r)
    tot = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    lines = [f"# {a.title}", "", "Command (from the repository root, on the GPU host):", "", "```"]
    lines += [c for c in a.command] + ["```", ""]
    lines += ["| kernel | calls | average ms | min ms | max ms | share |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("(anonymous namespace)::", "").split("(")[0]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
                     f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} | "
                     f"{100 * float(r['TotalDurationNs']) / tot:.1f}% |")
    if a.note:
        lines += ["", a.note]
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--command", action="append", default=[])
    s = sub.add_parser("stats")
    s.add_argument("--stats", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--command", action="append", default=[])
    s.add_argument("--note", default="")
    b = sub.add_parser("table")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", action="append", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--out", required=True)
    b.add_argument("--title", required=True)
    b.add_argument("--command", action="append", default=[])
    b.add_argument("--note", default="")
    c = sub.add_parser("counters")
    c.add_argument("--pmc", action="append", required=True)
    c.add_argument("--stats", required=True)
    c.add_argument("--kernel", action="append", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--command", action="append", default=[])
    c.add_argument("--note", default="")
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--simds", type=int, default=1024)
    a = ap.parse_args(argv)
    {"traffic": cmd_traffic, "table": cmd_table, "stats": cmd_stats, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())
