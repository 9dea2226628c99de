"""Turn two rocprofv3 counter runs of bench.py into the HBM-traffic record bench.py reports.

    python -m kv_cache_compressed_amd.pmc_summary FETCH.csv WRITE.csv --copy-mb 1024

FETCH.csv / WRITE.csv are the counter_collection.csv files of

    rocprofv3 --pmc FETCH_SIZE --output-format csv -- python3 bench.py --steps 2 --warmup 1 \\
        --no-cpu-baseline --eager --copy-mb 1024
    rocprofv3 --pmc WRITE_SIZE ... (same command)

The copy kernel (a plain device-to-device copy of --copy-mb MB, run by the HIP runtime's blit
kernel) calibrates each counter: its
true traffic is copy-mb MB read and copy-mb MB written, so scale = true bytes / counted bytes.
The draft attention kernel's counted bytes per dispatch are multiplied by that scale. Writes
profiles/draft_quant_c2_traffic.json (with the hash of the draft kernel source it was measured on)
and profiles/draft_quant_c2_traffic.md.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "kv_cache_compressed_amd", "csrc", "draft_quant.hip")
DRAFT = "draft_quant_kernel"
COPY_NAMES = ("copyBuffer", "copy_kernel")  # the runtime's blit kernel, torch's copy kernel


def per_dispatch(path: str, counter: str):
    """{kernel name: [KiB per dispatch]} for one counter (summed over the counter's instances)."""
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--copy-mb", type=int, required=True)
    ap.add_argument("--draft-bytes", type=float, default=205440000.0,
                    help="algorithmic bytes of one draft launch (bench.py's bytes_per_launch)")
    args = ap.parse_args()
    copy_bytes = args.copy_mb * 2 ** 20
    res = {}
    for counter, path in (("FETCH_SIZE", args.fetch_csv), ("WRITE_SIZE", args.write_csv)):
        d = per_dispatch(path, counter)
        copies = [v for name, vs in d.items() if any(c in name for c in COPY_NAMES) for v in vs]
        big = [v for v in copies if v * 1024 > 0.25 * copy_bytes]
        if not big:
            raise SystemExit(f"no copy dispatch of ~{args.copy_mb} MB found for {counter}")
        scale = copy_bytes / (statistics.median(big) * 1024)
        drafts = [v for name, vs in d.items() if DRAFT in name for v in vs]
        if not drafts:
            raise SystemExit(f"no {DRAFT} dispatch found for {counter}")
        res[counter] = {"copy_kib_median": statistics.median(big), "scale": scale,
                        "draft_kib_median": statistics.median(drafts), "draft_dispatches": len(drafts),
                        "draft_bytes_scaled": statistics.median(drafts) * 1024 * scale}
    fetch = res["FETCH_SIZE"]["draft_bytes_scaled"]
    write = res["WRITE_SIZE"]["draft_bytes_scaled"]
    rec = {"kernel": DRAFT, "workload": "c2 draft step (batch 8, 8 kv heads, 32640 quantised tokens, 2-bit)",
           "hbm_bytes_per_launch": round(fetch + write), "fetch_bytes": round(fetch),
           "write_bytes": round(write), "algorithmic_bytes": args.draft_bytes,
           "traffic_over_algorithmic": round((fetch + write) / args.draft_bytes, 4),
           "counters": res,
           "kernel_source_sha256_16": hashlib.sha256(open(SRC, "rb").read()).hexdigest()[:16]}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    json.dump(rec, open(os.path.join(ROOT, "profiles", "draft_quant_c2_traffic.json"), "w"), indent=1)
    md = [
        "# HBM traffic of the draft attention kernel (Llama-3.1-8B-shaped layer, batch 8, 32K context, KIVI 2-bit)\n",
        "Commands (repository root on one MI355X, `cd /tmp && export TMPDIR=/tmp` first), one counter per run:\n",
        "```",
        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <f> -o f -- python3 <repo>/bench.py --steps 2 --warmup 1 --no-cpu-baseline --eager --copy-mb %d" % args.copy_mb,
        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <w> -o w -- python3 <repo>/bench.py --steps 2 --warmup 1 --no-cpu-baseline --eager --copy-mb %d" % args.copy_mb,
        "python -m kv_cache_compressed_amd.pmc_summary <f>/f_counter_collection.csv <w>/w_counter_collection.csv --copy-mb %d" % args.copy_mb,
        "```\n",
        "Each counter is scaled by what it reads for a plain device copy of %d MB (true traffic: %d MB read, %d MB written).\n" % (args.copy_mb, args.copy_mb, args.copy_mb),
        "| counter | copy kernel KiB (median) | scale | draft kernel KiB per dispatch (median, %d dispatches) | scaled bytes |" % res["FETCH_SIZE"]["draft_dispatches"],
        "|---|---:|---:|---:|---:|",
    ]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        r = res[c]
        md.append(f"| {c} | {r['copy_kib_median']:.0f} | {r['scale']:.4f} | {r['draft_kib_median']:.0f} | {r['draft_bytes_scaled']:.0f} |")
    md.append("")
    md.append(f"HBM bytes per draft launch: {fetch + write:.0f} (algorithmic {args.draft_bytes:.0f}; ratio {(fetch + write) / args.draft_bytes:.3f}). "
              f"Kernel source hash: `{rec['kernel_source_sha256_16']}`.")
    open(os.path.join(ROOT, "profiles", "draft_quant_c2_traffic.md"), "w").write("\n".join(md) + "\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
