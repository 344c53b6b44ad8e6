"""Summaries of rocprofv3 output for the profiles/ folder.

Two summaries are produced from rocprofv3's CSV files:

* ``stats``: per-kernel call counts and durations from a ``--kernel-trace --stats``
  run (``*_kernel_stats.csv``), written as a text table.
* ``pmc``: per-dispatch means of any counters of ``--pmc`` runs for the kernels that
  match a pattern, with MFMA-busy, wait and LDS-conflict ratios.
* ``traffic``: HBM bytes per benchmark step from two ``--pmc`` runs, one with
  ``FETCH_SIZE`` and one with ``WRITE_SIZE`` (KiB per dispatch). Both runs include
  ``bench.py --copy-calib``, whose plain 512 MiB device copies calibrate the
  counters: each counter is scaled by 512 MiB divided by what it reads for one such
  copy. The result goes to ``traffic.json``, keyed by the hash of the kernel
  sources so that ``bench.py`` ignores it once a kernel changes.

    python profsum.py stats STATS_CSV OUT_TXT --command CMD
    python profsum.py traffic FETCH_CSV WRITE_CSV OUT_JSON OUT_TXT \
        --command CMD
    python profsum.py pmc KERNEL_REGEX OUT_TXT COUNTER_CSV [COUNTER_CSV ...] --command CMD
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))

# kernels that make up one step of each workload (matched on the demangled name)
STEP_KERNELS = {
    "gla_bf16_b2h8_n2048_d128": [r"gla_prep_kernel<", r"gla_chain_kernel<(true|false), \d>"],
    "ssd_bf16_b2h32_n4096_dk128_dv64": [r"ssd_chain_kernel<"],
    "kath_bf16_b1h16_n32768_dk128_dv64": [r"kath_chain_kernel<", r"kath_scan_kernel"],
    "gdn_bf16_b4h16_n8192_d128": [r"gdn_prep_kernel<", r"gdn_fwd_kernel<"],
    "kda_bf16_b4h16_n8192_d128": [r"kda_prep_kernel<", r"kda_fwd_kernel<"],
    "kath_f32_n256_d16": [r"prefill_valu_kernel<0,"],
    "selscan_bf16_b2_t4096_d2048_n128": [r"selective_scan_kernel<128,"],
    "selscan_bf16_b2_t4096_d2048_n16": [r"selective_scan_kernel<16,"],
    "decode_gdn_256x32_d128": [r"decode_(persist_)?kernel<2,"],
    "decode_gla_256x32_d128": [r"decode_(persist_)?kernel<1,"],
    "decode_kda_256x32_d128": [r"decode_(persist_)?kernel<3,"],
    "decode_ssd_256x64_dk128_dv64": [r"decode_(persist_)?kernel<4,"],
}
COPY_BYTES = 512 << 20


def short(name: str) -> str:
    name = name.replace("void la::(anonymous namespace)::", "")
    name = name.replace("(la::(anonymous namespace)::", "(")
    return name


def stats(csv_path: str, out_txt: str, command: str) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {command}", "#",
             f"# {'kernel':<64} {'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
    for r in rows:
        lines.append(f"  {short(r['Name'])[:64]:<64} {int(r['Calls']):>7} "
                     f"{float(r['AverageNs']) / 1e3:>10.2f} {float(r['MinNs']) / 1e3:>10.2f} "
                     f"{float(r['MaxNs']) / 1e3:>10.2f} {float(r['Percentage']):>6.2f}")
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


def per_dispatch(csv_path: str, counter: str):
    """{kernel name: [value per dispatch, ...]} of one counter (summed over instances)."""
    acc = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        key = r["Dispatch_Id"]
        acc[key] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for key, v in acc.items():
        out[names[key]].append(v)
    return out


def calibration(values) -> float:
    copies = [v for name, vs in values.items() if "copyBuffer" in name for v in vs]
    if not copies:
        raise SystemExit("no device copy dispatch found: run bench.py with --copy-calib")
    top = max(copies)
    return (COPY_BYTES / 1024.0) / top


def traffic(fetch_csv: str, write_csv: str, out_json: str, out_txt: str, command: str) -> None:
    sys.path.insert(0, ROOT)
    from bench import kernel_source_hash
    f = per_dispatch(fetch_csv, "FETCH_SIZE")
    w = per_dispatch(write_csv, "WRITE_SIZE")
    cf, cw = calibration(f), calibration(w)
    res = {"kernel_source_hash": kernel_source_hash(), "unit": "bytes",
           "calibration": {"copy_bytes": COPY_BYTES, "fetch_factor": cf, "write_factor": cw},
           "workloads": {}}
    lines = [f"# HBM traffic per step from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch)",
             f"# command: {command}",
             f"# calibration: a 512 MiB device copy reads FETCH x {cf:.4f}, WRITE x {cw:.4f}",
             "#", f"# {'workload / kernel':<60} {'fetch_MB':>10} {'write_MB':>10}"]
    for wl, pats in STEP_KERNELS.items():
        tot_f = tot_w = 0.0
        found = False
        kern = {}
        for pat in pats:
            for name, vs in f.items():
                if re.search(pat, short(name)):
                    wv = w.get(name, [0.0])
                    fb = sum(vs) / len(vs) * 1024.0 * cf
                    wb = sum(wv) / len(wv) * 1024.0 * cw
                    kern[short(name)] = {"fetch_bytes": fb, "write_bytes": wb, "dispatches": len(vs)}
                    tot_f += fb
                    tot_w += wb
                    found = True
        if not found:
            continue
        res["workloads"][wl] = {"hbm_bytes_per_step": tot_f + tot_w, "fetch_bytes": tot_f,
                                "write_bytes": tot_w, "kernels": kern}
        lines.append(f"  {wl:<60} {tot_f / 1e6:>10.2f} {tot_w / 1e6:>10.2f}")
        for k, v in kern.items():
            lines.append(f"    {k[:58]:<58} {v['fetch_bytes'] / 1e6:>10.2f} "
                         f"{v['write_bytes'] / 1e6:>10.2f}")
    with open(out_json, "w") as fh:
        json.dump(res, fh, indent=1)
    with open(out_txt, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def pmc(csv_paths, kernel_pat: str, out_txt: str, command: str) -> None:
    """Per-dispatch averages of every counter in the given counter_collection CSVs, for the
    kernels whose demangled name matches kernel_pat, with a few ratios derived from them."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in csv_paths:
        acc = collections.defaultdict(float)
        names = {}
        for r in csv.DictReader(open(path)):
            if not re.search(kernel_pat, short(r["Kernel_Name"])):
                continue
            key = (r["Dispatch_Id"], r["Counter_Name"])
            acc[key] += float(r["Counter_Value"])
            names[key] = short(r["Kernel_Name"])
        for (disp, cname), v in acc.items():
            vals[names[(disp, cname)]][cname].append(v)
    lines = ["# rocprofv3 counters, mean per dispatch", f"# command: {command}", "#"]
    for kern, cs in vals.items():
        lines.append(f"  {kern}")
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        for c in sorted(m):
            lines.append(f"    {c:<32} {m[c]:>18.1f}   ({len(cs[c])} dispatches)")
        def ratio(label, a, b):
            if a in m and b in m and m[b] > 0:
                lines.append(f"    {label:<32} {m[a] / m[b]:>18.4f}")
        ratio("MFMA busy / busy cycles", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES")
        ratio("LDS wait / wave cycles", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES")
        ratio("any wait / wave cycles", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")
        ratio("LDS bank conflict / LDS active", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS")
        ratio("VMEM active / wave cycles", "SQ_ACTIVE_INST_VMEM", "SQ_WAVE_CYCLES")
    with open(out_txt, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("out_json")
    t.add_argument("out_txt")
    t.add_argument("--command", required=True)
    c = sub.add_parser("pmc")
    c.add_argument("kernel", help="regular expression on the demangled kernel name")
    c.add_argument("out")
    c.add_argument("csv", nargs="+")
    c.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.what == "stats":
        stats(a.csv, a.out, a.command)
    elif a.what == "pmc":
        pmc(a.csv, a.kernel, a.out, a.command)
    else:
        traffic(a.fetch_csv, a.write_csv, a.out_json, a.out_txt, a.command)


if __name__ == "__main__":
    main()
