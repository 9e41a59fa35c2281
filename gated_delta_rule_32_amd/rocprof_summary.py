"""Summarise rocprofv3 CSV output for libkda kernels.

Usage:
  python -m gated_delta_rule_32_amd.rocprof_summary trace  DIR [--match SUBSTR]
      per-kernel duration statistics from a `--kernel-trace --stats
      --output-format csv` run (reads *_kernel_stats.csv / *_kernel_trace.csv)
  python -m gated_delta_rule_32_amd.rocprof_summary counters DIR [--match SUBSTR]
      per-kernel mean of every counter from a `--pmc ... --output-format csv`
      run (reads *_counter_collection.csv)
  python -m gated_delta_rule_32_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR
      --match SUBSTR --copy-fetch CF_DIR --copy-write CW_DIR --copy-bytes N
      HBM bytes per launch of the matching kernel: FETCH_SIZE and WRITE_SIZE
      (KiB per dispatch) scaled by what the same counters read for a plain
      copy kernel that reads and writes N bytes.
  python -m gated_delta_rule_32_amd.rocprof_summary mfma PMC_DIR [PMC_DIR ...]
      --match SUBSTR --trace TRACE_DIR [--record KEY --src FILE --source NAME]
      counter-derived MFMA and LDS figures of the matching kernel from `--pmc`
      runs holding SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES,
      GRBM_GUI_ACTIVE, SQ_INSTS_LDS and SQ_LDS_BANK_CONFLICT (any split over
      the runs), with the mean kernel duration from a kernel-trace run:
        executed bf16 MFMA FLOPs = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16
        MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x CUs x 4)
          (rocprofv3 reports GRBM_GUI_ACTIVE summed over the 8 XCDs; the
          busy fraction takes its per-XCD value, as the MfmaUtil expression's
          reduce(GRBM_GUI_ACTIVE, max) does)
        LDS bank-conflict cycles per LDS instruction
      With --record, the figures are also stored under KEY in
      profiles/counters.json together with the sha256 of FILE.
Output is Markdown on stdout.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import statistics
import sys
from collections import defaultdict


def _rows(d, pattern):
    files = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def trace(d, match=None):
    rows = _rows(d, "*kernel_trace.csv")
    per = defaultdict(list)
    for r in rows:
        name = r.get("Kernel_Name", "")
        if match and match not in name:
            continue
        try:
            per[name].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        except (KeyError, ValueError):
            continue
    print("| kernel | calls | mean us | median us | min us | max us | total ms |")
    print("|---|---|---|---|---|---|---|")
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) < 90 else name[:87] + "..."
        print(f"| `{short}` | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} "
              f"| {min(v):.2f} | {max(v):.2f} | {sum(v) / 1e3:.3f} |")
    return per


def counters(d, match=None):
    rows = _rows(d, "*counter_collection.csv")
    per = defaultdict(lambda: defaultdict(list))
    for r in rows:
        name = r.get("Kernel_Name", "")
        if match and match not in name:
            continue
        per[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = {}
    for name, cs in per.items():
        print(f"### `{name[:100]}`\n")
        print("| counter | dispatches | mean per dispatch |")
        print("|---|---|---|")
        out[name] = {}
        for c, v in sorted(cs.items()):
            m = statistics.mean(v)
            out[name][c] = m
            print(f"| {c} | {len(v)} | {m:.1f} |")
        print()
    return out


def _mean_counter(d, counter, match):
    vals = []
    for r in _rows(d, "*counter_collection.csv"):
        if match in r.get("Kernel_Name", "") and r["Counter_Name"] == counter:
            vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {match!r} in {d}")
    return statistics.mean(vals), len(vals)


def traffic(fetch_dir, write_dir, match, cf_dir, cw_dir, copy_bytes, copy_match):
    f_kib, nf = _mean_counter(fetch_dir, "FETCH_SIZE", match)
    w_kib, nw = _mean_counter(write_dir, "WRITE_SIZE", match)
    cf_kib, _ = _mean_counter(cf_dir, "FETCH_SIZE", copy_match)
    cw_kib, _ = _mean_counter(cw_dir, "WRITE_SIZE", copy_match)
    sf = copy_bytes / (cf_kib * 1024.0)
    sw = copy_bytes / (cw_kib * 1024.0)
    fetch_b = f_kib * 1024.0 * sf
    write_b = w_kib * 1024.0 * sw
    print(f"| quantity | value |\n|---|---|")
    print(f"| kernel match | `{match}` ({nf} / {nw} dispatches) |")
    print(f"| FETCH_SIZE raw (KiB/dispatch) | {f_kib:.1f} |")
    print(f"| WRITE_SIZE raw (KiB/dispatch) | {w_kib:.1f} |")
    print(f"| copy kernel FETCH_SIZE / WRITE_SIZE (KiB) for {copy_bytes} B each way | {cf_kib:.1f} / {cw_kib:.1f} |")
    print(f"| scale factors fetch / write | {sf:.4f} / {sw:.4f} |")
    print(f"| HBM read bytes per launch | {fetch_b:.4e} |")
    print(f"| HBM write bytes per launch | {write_b:.4e} |")
    print(f"| HBM bytes per launch (read + write) | {fetch_b + write_b:.4e} |")
    return fetch_b + write_b


N_CU = 256          # MI355X compute units (4 SIMDs each)
N_XCD = 8           # accelerator complex dies (GRBM_GUI_ACTIVE is summed over them)


def mfma(pmc_dirs, match, trace_dir, key=None, src=None, source=None):
    import hashlib
    import json
    vals = {}
    for d in pmc_dirs:
        for r in _rows(d, "*counter_collection.csv"):
            if match in r.get("Kernel_Name", ""):
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    mean = {c: statistics.mean(v) for c, v in vals.items()}
    durs = []
    for r in _rows(trace_dir, "*kernel_trace.csv"):
        if match in r.get("Kernel_Name", ""):
            durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if not durs or "SQ_INSTS_VALU_MFMA_MOPS_BF16" not in mean:
        raise SystemExit(f"no trace rows or MFMA counters for kernels matching {match!r}")
    us = statistics.mean(durs)
    flops = 512.0 * mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
    rec = {"kernel_us": round(us, 2), "mfma_bf16_flops": flops,
           "mfma_tflops": round(flops / us / 1e6, 2)}
    print("| quantity | value |\n|---|---|")
    print(f"| kernel match | `{match}` ({len(durs)} traced dispatches) |")
    for c in sorted(mean):
        print(f"| {c} per dispatch | {mean[c]:.4g} ({len(vals[c])} dispatches) |")
    print(f"| mean kernel duration (trace) | {us:.2f} us |")
    print(f"| executed bf16 MFMA FLOPs per dispatch (512 x MOPS) | {flops:.4e} |")
    print(f"| executed bf16 MFMA rate | {flops / us / 1e6:.1f} TFLOP/s |")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in mean and "GRBM_GUI_ACTIVE" in mean:
        gui = mean["GRBM_GUI_ACTIVE"] / N_XCD
        busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * N_CU * 4)
        rec["mfma_busy_frac"] = round(busy, 4)
        rec["gpu_clock_ghz"] = round(gui / us / 1e3, 3)
        print(f"| GPU busy cycles per XCD (GRBM_GUI_ACTIVE / {N_XCD}) | {gui:.4g} ({gui / us / 1e3:.2f} GHz over the traced duration) |")
        print(f"| MFMA busy fraction, BUSY_CYCLES / (GUI_ACTIVE / {N_XCD} x {N_CU} x 4) | {busy:.4f} |")
    if "SQ_LDS_BANK_CONFLICT" in mean and mean.get("SQ_INSTS_LDS"):
        per = mean["SQ_LDS_BANK_CONFLICT"] / mean["SQ_INSTS_LDS"]
        rec["lds_bank_conflict_per_lds_inst"] = round(per, 3)
        print(f"| LDS bank-conflict cycles per LDS instruction | {per:.3f} |")
    if key:
        with open(src, "rb") as f:
            rec["src_sha256_16"] = hashlib.sha256(f.read()).hexdigest()[:16]
        rec["source"] = source
        path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "profiles", "counters.json")
        try:
            with open(path) as f:
                allr = json.load(f)
        except (OSError, ValueError):
            allr = {}
        allr[key] = rec
        with open(path, "w") as f:
            json.dump(allr, f, indent=1, sort_keys=True)
            f.write("\n")
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace"); t.add_argument("dir"); t.add_argument("--match")
    c = sub.add_parser("counters"); c.add_argument("dir"); c.add_argument("--match")
    x = sub.add_parser("traffic")
    x.add_argument("fetch_dir"); x.add_argument("write_dir")
    x.add_argument("--match", required=True)
    x.add_argument("--copy-fetch", required=True); x.add_argument("--copy-write", required=True)
    x.add_argument("--copy-bytes", type=float, required=True)
    x.add_argument("--copy-match", default="copy")
    m = sub.add_parser("mfma")
    m.add_argument("pmc_dirs", nargs="+")
    m.add_argument("--match", required=True); m.add_argument("--trace", required=True)
    m.add_argument("--record"); m.add_argument("--src"); m.add_argument("--source")
    a = ap.parse_args(argv)
    if a.cmd == "mfma":
        mfma(a.pmc_dirs, a.match, a.trace, a.record, a.src, a.source)
        return 0
    if a.cmd == "trace":
        trace(a.dir, a.match)
    elif a.cmd == "counters":
        counters(a.dir, a.match)
    else:
        traffic(a.fetch_dir, a.write_dir, a.match, a.copy_fetch, a.copy_write, a.copy_bytes,
                a.copy_match)
    return 0


if __name__ == "__main__":
    sys.exit(main())
