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
    names = counter_names(args.csv)
    data = {c: per_dispatch(args.csv, c) for c in names}
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
          f"python -m kv_cache_compressed_amd.pmc_summary counters <out>/m_counter_collection.csv "
          f"--name {args.name} --kernels {' '.join(args.kernels)}", "```\n",
          "Medians per dispatch. `GRBM_GUI_ACTIVE` is summed over the 8 XCDs; matrix-core "
          "utilisation = `SQ_VALU_MFMA_BUSY_CYCLES` / (`GRBM_GUI_ACTIVE` / 8 x 1024 SIMDs).\n",
          "| kernel | dispatches | " + " | ".join(f"`{c}`" for c in names) + " | MFMA busy |",
          "|---|---:|" + "---:|" * len(names) + "---:|"]
    for k, nd, med, util in rows:
        cells = " | ".join(f"{med[c]:,.0f}" if c in med else "" for c in names)
        md.append(f"| `{k}` | {nd} | {cells} | {'' if util is None else f'{100 * util:.1f}%'} |")
    md.append("")
    if args.note:
        md.append(args.note + "\n")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    open(os.path.join(ROOT, "profiles", f"{args.name}_counters.md"), "w").write("\n".join(md))
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
    c.add_argument("csv")
    c.add_argument("--name", required=True)
    c.add_argument("--kernels", nargs="+", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--note", default="")
    args = ap.parse_args()
    traffic(args) if args.cmd == "traffic" else counters(args)


if __name__ == "__main__":
    main()
