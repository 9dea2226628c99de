"""Turn rocprofv3 counter runs of bench.py into the summaries kept under profiles/.

HBM traffic of one kernel (two runs, one counter each, both with --copy-mb so a plain device copy of
known size calibrates the counters):

    python -m kv_cache_compressed_amd.pmc_summary traffic FETCH.csv WRITE.csv --copy-mb 1024 \\
        --kernel draft_quant_kernel --bytes 205440000 --name draft_quant_c2 \\
        --src kv_cache_compressed_amd/csrc/draft_quant.hip --workload "..." --command "..."

FETCH.csv / WRITE.csv are the counter_collection.csv files of

    rocprofv3 --pmc FETCH_SIZE --output-format csv -- python3 bench.py ... --copy-mb 1024
    rocprofv3 --pmc WRITE_SIZE ... (same command)

The copy kernel (the HIP runtime's blit kernel or torch's copy kernel) moves copy-mb MB in and
copy-mb MB out, so scale = true bytes / counted bytes for each counter; the kernel's counted bytes
per dispatch (median) are multiplied by that scale. Writes profiles/<name>_traffic.json (with the
hash of the kernel's source it was measured on, which bench.py checks before reporting it) and
profiles/<name>_traffic.md.

A counter_collection.csv summed over counter instances (one row per dispatch and counter, the
columns the other subcommands read), to keep the files of long runs small:

    python -m kv_cache_compressed_amd.pmc_summary reduce RAW.csv OUT.csv

Kernel time summary of a `rocprofv3 --kernel-trace --stats --output-format csv` run:

    python -m kv_cache_compressed_amd.pmc_summary stats X_kernel_stats.csv --name c2_round \
        --title "..." --command "..." [--note "..."]

writes profiles/<name>_kernel_stats.md (kernels by total time: calls, average / min / max
microseconds, share of GPU time).

Per-kernel medians of any counters (e.g. the matrix-core pass):

    python -m kv_cache_compressed_amd.pmc_summary counters M.csv --name verify_c2_mfma \\
        --kernels verify_bf16_kernel draft_quant_kernel --title "..." --command "..."

writes profiles/<name>_counters.md with one row per kernel: dispatches, every counter's median per
dispatch, and the matrix-core utilisation SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x
SIMDs) when both counters are present (GRBM_GUI_ACTIVE is summed over the 8 XCDs).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_NAMES = ("copyBuffer", "copy_kernel")  # the runtime's blit kernel, torch's copy kernel
XCDS, SIMDS = 8, 1024


def per_dispatch(path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter (summed over the counter's instances)."""
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (_, name), v in sorted(acc.items()):
        out.setdefault(name, []).append(v)
    return out


def counter_names(path: str):
    return sorted({r["Counter_Name"] for r in csv.DictReader(open(path))})


def src_hash(src: str) -> str:
    return hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()[:16]


def traffic(args):
    copy_bytes = args.copy_mb * 2 ** 20
    res = {}
    for counter, path in (("FETCH_SIZE", args.fetch_csv), ("WRITE_SIZE", args.write_csv)):
        d = per_dispatch(path, counter)
        copies = [v for name, vs in d.items() if any(c in name for c in COPY_NAMES) for v in vs]
        big = [v for v in copies if v * 1024 > 0.25 * copy_bytes]
        if not big:
            raise SystemExit(f"no copy dispatch of ~{args.copy_mb} MB found for {counter}")
        scale = copy_bytes / (statistics.median(big) * 1024)
        mine = [v for name, vs in d.items() if args.kernel in name for v in vs]
        if not mine:
            raise SystemExit(f"no {args.kernel} dispatch found for {counter}")
        res[counter] = {"copy_kib_median": statistics.median(big), "scale": scale,
                        "kernel_kib_median": statistics.median(mine), "dispatches": len(mine),
                        "bytes_scaled": statistics.median(mine) * 1024 * scale}
    fetch = res["FETCH_SIZE"]["bytes_scaled"]
    write = res["WRITE_SIZE"]["bytes_scaled"]
    rec = {"kernel": args.kernel, "workload": args.workload,
           "hbm_bytes_per_launch": round(fetch + write), "fetch_bytes": round(fetch),
           "write_bytes": round(write), "algorithmic_bytes": args.bytes,
           "traffic_over_algorithmic": round((fetch + write) / args.bytes, 4),
           "counters": res, "kernel_source": args.src,
           "kernel_source_sha256_16": src_hash(args.src)}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    json.dump(rec, open(os.path.join(ROOT, "profiles", f"{args.name}_traffic.json"), "w"), indent=1)
    md = [
        f"# HBM traffic of `{args.kernel}`: {args.workload}\n",
        "Commands (repository root on one MI355X, `cd /tmp && export TMPDIR=/tmp` first), one counter per run:\n",
        "```",
        args.command.replace("<COUNTER>", "FETCH_SIZE"),
        args.command.replace("<COUNTER>", "WRITE_SIZE"),
        f"python -m kv_cache_compressed_amd.pmc_summary traffic <f>/f_counter_collection.csv "
        f"<w>/w_counter_collection.csv --copy-mb {args.copy_mb} --kernel {args.kernel} "
        f"--bytes {args.bytes:.0f} --name {args.name} --src {args.src}",
        "```\n",
        f"Each counter is scaled by what it reads for a plain device copy of {args.copy_mb} MB (true "
        f"traffic: {args.copy_mb} MB read, {args.copy_mb} MB written).\n",
        f"| counter | copy kernel KiB (median) | scale | kernel KiB per dispatch (median, "
        f"{res['FETCH_SIZE']['dispatches']} dispatches) | scaled bytes |",
        "|---|---:|---:|---:|---:|",
    ]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        r = res[c]
        md.append(f"| {c} | {r['copy_kib_median']:.0f} | {r['scale']:.4f} | {r['kernel_kib_median']:.0f} | "
                  f"{r['bytes_scaled']:.0f} |")
    md.append("")
    md.append(f"HBM bytes per launch: {fetch + write:.0f} (algorithmic {args.bytes:.0f}; ratio "
              f"{(fetch + write) / args.bytes:.3f}). Kernel source `{args.src}`, hash "
              f"`{rec['kernel_source_sha256_16']}`.")
    open(os.path.join(ROOT, "profiles", f"{args.name}_traffic.md"), "w").write("\n".join(md) + "\n")
    print(json.dumps(rec, indent=1))


def counters(args):
    data = {}
    for path in args.csv:  # one file per counter pass; a counter read in several passes: the first
        for c in counter_names(path):
            data.setdefault(c, per_dispatch(path, c))
    names = sorted(data)
    rows = []
    for k in args.kernels:
        med, nd = {}, 0
        for c in names:
            vs = [v for name, lst in data[c].items() if k in name for v in lst]
            if vs:
                med[c] = statistics.median(vs)
                nd = max(nd, len(vs))
        if not med:
            continue
        util = None
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med and "GRBM_GUI_ACTIVE" in med:
            util = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (med["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
        rows.append((k, nd, med, util))
    md = [f"# {args.title}\n",
          "Command (repository root on one MI355X, `cd /tmp && export TMPDIR=/tmp` first):\n",
          "```", args.command,
          f"python -m kv_cache_compressed_amd.pmc_summary counters <pass csv> ... "
          f"--name {args.name} --kernels {' '.join(args.kernels)}", "```\n",
          "Medians per dispatch, one row per counter (a rocprofv3 run collects one pass of counters; "
          "the passes are separate runs of the same command). `GRBM_GUI_ACTIVE` is summed over the "
          "8 XCDs; matrix-core utilisation = `SQ_VALU_MFMA_BUSY_CYCLES` / (`GRBM_GUI_ACTIVE` / 8 x "
          "1024 SIMDs); the `SQ_WAIT_*` / `SQ_ACTIVE_*` shares are of `SQ_WAVE_CYCLES`.\n",
          "| counter | " + " | ".join(f"`{k}` ({nd} dispatches)" for k, nd, _, _ in rows) + " |",
          "|---|" + "---:|" * len(rows)]
    for c in names:
        cells = []
        for _, _, med, _ in rows:
            v = med.get(c)
            cell = "" if v is None else f"{v:,.0f}"
            if v is not None and c.startswith(("SQ_WAIT", "SQ_ACTIVE")) and med.get("SQ_WAVE_CYCLES"):
                cell += f" ({100 * v / med['SQ_WAVE_CYCLES']:.1f}%)"
            cells.append(cell)
        md.append(f"| `{c}` | " + " | ".join(cells) + " |")
    md.append("| MFMA busy | " + " | ".join("" if u is None else f"{100 * u:.1f}%" for _, _, _, u in rows) + " |")
    md.append("")
    if args.note:
        md.append(args.note + "\n")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    open(os.path.join(ROOT, "profiles", f"{args.name}_counters.md"), "w").write("\n".join(md))
    print("\n".join(md))


def reduce(args):
    acc, names = {}, {}
    for r in csv.DictReader(open(args.raw)):
        key = (int(r["Dispatch_Id"]), r["Counter_Name"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        names[int(r["Dispatch_Id"])] = r["Kernel_Name"]
    with open(args.out, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for (d, c), v in sorted(acc.items()):
            w.writerow([d, names[d], c, v])


def short_name(name: str, width: int = 90) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("vc::", "").replace("void ", "")
    return n if len(n) <= width else n[:width - 3] + "..."


def stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    md = [f"# {args.title}\n",
          "Command (repository root on one MI355X, `cd /tmp && export TMPDIR=/tmp` first):\n",
          "```", args.command,
          f"python -m kv_cache_compressed_amd.pmc_summary stats <out>/<x>_kernel_stats.csv --name {args.name}",
          "```\n"]
    if args.note:
        md.append(args.note + "\n")
    md += ["| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows[:args.top]:
        md.append(f"| `{short_name(r['Name'])}` | {int(r['Calls'])} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                  f"{100 * float(r['TotalDurationNs']) / total:.2f} |")
    md.append("")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    open(os.path.join(ROOT, "profiles", f"{args.name}_kernel_stats.md"), "w").write("\n".join(md))
    print("\n".join(md))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--copy-mb", type=int, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--bytes", type=float, required=True, help="algorithmic bytes of one launch")
    t.add_argument("--name", required=True)
    t.add_argument("--src", required=True, help="kernel source, relative to the repository root")
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True, help="the profiled command, <COUNTER> for the counter")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--name", required=True)
    c.add_argument("--kernels", nargs="+", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--note", default="")
    r = sub.add_parser("reduce")
    r.add_argument("raw")
    r.add_argument("out")
    st = sub.add_parser("stats")
    st.add_argument("csv")
    st.add_argument("--name", required=True)
    st.add_argument("--title", required=True)
    st.add_argument("--command", required=True)
    st.add_argument("--note", default="")
    st.add_argument("--top", type=int, default=16)
    args = ap.parse_args()
    {"traffic": traffic, "counters": counters, "reduce": reduce, "stats": stats}[args.cmd](args)


if __name__ == "__main__":
    main()
