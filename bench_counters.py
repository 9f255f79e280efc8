#!/usr/bin/env python3
"""Summaries of rocprofv3 output for profiles/ (text only; bench.py reads
profiles/traffic.json).

  python bench_counters.py stats DIR OUT.md --command CMD
      kernel-trace statistics (rocprofv3 --kernel-trace --stats, csv) of
      every kernel, with bench.py's dominant kernels marked.
  python bench_counters.py traffic FETCH_DIR WRITE_DIR --copy-mib M --command CMD
      HBM bytes per launch of each workload's dominant kernel from one
      FETCH_SIZE and one WRITE_SIZE run (rocprofv3 --pmc, csv), scaled by
      what the same counters read for the plain M MiB device copy those runs
      start with; writes profiles/traffic.json and
      profiles/hbm_traffic_dominant_kernels.md.
  python bench_counters.py pmc OUT.md --kernel PREFIX --command CMD DIR [DIR ...]
      per-dispatch means of every counter collected for one kernel.
  python bench_counters.py benchline LINE.json OUT.md --command CMD
      a table of one bench.py JSON line (every workload), with the line itself.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def _name(k):
    k = k[5:] if k.startswith("void ") else k
    return k.replace("cnf::(anonymous namespace)::", "").replace("cnf::", "")


def _find(d, suffix):
    fs = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not fs:
        raise SystemExit(f"no *{suffix} under {d}")
    return fs


def _counters(dirs, wanted=None):
    """{kernel: {counter: [value per dispatch]}}"""
    per = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        for f in _find(d, "counter_collection.csv"):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    c = r["Counter_Name"]
                    if wanted is None or c in wanted:
                        per[_name(r["Kernel_Name"])][c].append(float(r["Counter_Value"]))
    return per


def stats(d, out, command):
    import bench
    rows = []
    for f in _find(d, "kernel_stats.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    # per-dispatch durations from the kernel trace, for the median
    dur = defaultdict(list)
    for f in _find(d, "kernel_trace.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                dur[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    dom = {v[0]: k for k, v in bench.DOMINANT.items()}
    L = ["# Kernel statistics, every workload of bench.py (rocprofv3 --kernel-trace --stats)", "",
         "Command (run from /tmp on the MI355X box, repository at $R):", "", "```", command, "```",
         "", "Dominant kernels (the ones bench.py times with cnf_forward_timed) are marked with the "
         "workload they serve.", "",
         "| kernel | calls | avg us | median us | min us | max us | % of GPU time | dominant in |",
         "|---|---:|---:|---:|---:|---:|---:|---|"]
    for r in rows:
        nm = _name(r["Name"])
        ws = sorted({w for p, w in dom.items() if nm.startswith(p)})
        short = nm if len(nm) <= 110 else nm[:110] + "..."
        ds = sorted(dur.get(r["Name"], [])) or [float("nan")]
        med = (ds[(len(ds) - 1) // 2] + ds[len(ds) // 2]) / 2
        L.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {med / 1e3:.1f} | "
                 f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                 f"{float(r['Percentage']):.1f} | {', '.join(ws)} |")
    with open(out, "w") as fh:
        fh.write("\n".join(L) + "\n")


def traffic(fetch_dir, write_dir, mib, command):
    import bench
    import cnf_inputs
    fe = {k: v["FETCH_SIZE"] for k, v in _counters([fetch_dir], {"FETCH_SIZE"}).items()}
    wr = {k: v["WRITE_SIZE"] for k, v in _counters([write_dir], {"WRITE_SIZE"}).items()}
    copyk = [k for k in fe if "UnaryFunctor" in k or "MulFunctor" in k]
    if not copyk:
        raise SystemExit("no copy-calibration kernel in the FETCH_SIZE run")
    ck = max(copyk, key=lambda k: sum(fe[k]) / len(fe[k]))
    cb = mib * (1 << 20)
    fk, wk = sum(fe[ck]) / len(fe[ck]), sum(wr[ck]) / len(wr[ck])
    fs, ws = cb / 1024 / fk, cb / 1024 / wk
    out = {"_calibration": {"kernel": ck[:120], "copy_bytes": cb, "fetch_kib_measured": fk,
                            "write_kib_measured": wk, "fetch_scale": fs, "write_scale": ws,
                            "command": command}}
    L = ["# HBM traffic of each workload's dominant kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
         "Commands (run from /tmp on the MI355X box, repository at $R), one counter per run:", "",
         "```", command, "```", "",
         f"Calibration: a plain elementwise copy of {mib} MiB (`{ck[:60]}`) reads {fk:.0f} KiB and "
         f"writes {wk:.0f} KiB by these counters, so counter values are scaled by {fs:.4f} (FETCH) "
         f"and {ws:.4f} (WRITE).  These are L2-miss bytes, so lines served by the MALL count too.", "",
         "Each workload's entry holds the digest of its dominant kernel's sources at measurement; "
         "bench.py reports the traffic only while the sources still match.", "",
         "| workload | dominant kernel | read MB / launch | written MB / launch | HBM MB / launch | "
         "algorithmic MB / launch | ratio |",
         "|---|---|---:|---:|---:|---:|---:|"]
    for name in cnf_inputs.WORKLOAD_ORDER:
        kern = bench.DOMINANT[name][0]
        ks = [k for k in fe if k.startswith(kern)]
        if len(ks) != 1:
            raise SystemExit(f"{name}: {len(ks)} kernels match {kern!r}")
        k = ks[0]
        f_, w_ = sum(fe[k]) / len(fe[k]), sum(wr[k]) / len(wr[k])
        hb = f_ * 1024 * fs + w_ * 1024 * ws
        ab = bench.algorithmic_bytes(cnf_inputs.workload(name))
        out[name] = {"kernel": kern, "kernel_source_digest": bench.kernel_source_digest(name),
                     "hbm_bytes_per_launch": hb, "fetch_kib_per_dispatch": f_,
                     "write_kib_per_dispatch": w_, "algorithmic_bytes": ab}
        L.append(f"| {name} | `{kern}` | {f_ * 1024 * fs / 1e6:.1f} | {w_ * 1024 * ws / 1e6:.1f} | "
                 f"{hb / 1e6:.1f} | {ab / 1e6:.1f} | {hb / ab:.2f} |")
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    with open(os.path.join(ROOT, "profiles", "hbm_traffic_dominant_kernels.md"), "w") as fh:
        fh.write("\n".join(L) + "\n")


def pmc(out, kernel, command, dirs):
    per = _counters(dirs)
    ks = [k for k in per if k.startswith(kernel)]
    if len(ks) != 1:
        raise SystemExit(f"{len(ks)} kernels match {kernel!r}: {ks[:5]}")
    d = per[ks[0]]
    L = [f"# Counters of `{kernel}` (rocprofv3 --pmc, per-dispatch means)", "",
         "Commands (run from /tmp on the MI355X box, repository at $R), one counter set per run:",
         "", "```", command, "```", "",
         "| counter | per dispatch | dispatches |", "|---|---:|---:|"]
    for c in sorted(d):
        v = d[c]
        L.append(f"| {c} | {sum(v) / len(v):.6g} | {len(v)} |")
    m = {c: sum(v) / len(v) for c, v in d.items()}
    if "GRBM_GUI_ACTIVE" in m:
        # GRBM_GUI_ACTIVE sums the 8 XCDs; SQ cycle counters are per wave or per
        # SIMD summed over the chip's 1024 SIMDs, ACTIVE/WAIT ones in quad-cycles
        cyc = m["GRBM_GUI_ACTIVE"] / 8
        simd = 1024 * cyc
        L += ["", f"Derived (MI355X: 8 XCDs, 256 CUs, 1024 SIMDs; {cyc:.4g} GPU cycles per dispatch):", ""]
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            L.append(f"- MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (1024 x cycles) = "
                     f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / simd:.3f}")
        if "SQ_ACTIVE_INST_VALU" in m:
            L.append(f"- VALU busy (incl. MFMA issue): 4 x SQ_ACTIVE_INST_VALU / (1024 x cycles) = "
                     f"{4 * m['SQ_ACTIVE_INST_VALU'] / simd:.3f}")
        if "SQ_WAIT_INST_ANY" in m and "SQ_WAVE_CYCLES" in m:
            L.append(f"- waves waiting on a dependency: SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES = "
                     f"{m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.3f}")
        if "SQ_WAIT_ANY" in m and "SQ_WAVE_CYCLES" in m:
            L.append(f"- waves waiting for anything: SQ_WAIT_ANY / SQ_WAVE_CYCLES = "
                     f"{m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.3f}")
        if "TA_TA_BUSY" in m:
            L.append(f"- texture addresser busy: TA_TA_BUSY / (256 x cycles) = "
                     f"{m['TA_TA_BUSY'] / (256 * cyc):.3f}")
        if "SQ_INSTS_MFMA" in m and "SQ_WAVES" in m:
            L.append(f"- per wave: {m['SQ_INSTS_MFMA'] / m['SQ_WAVES']:.4g} MFMA, "
                     f"{m.get('SQ_INSTS_VALU', 0) / m['SQ_WAVES']:.4g} VALU, "
                     f"{m.get('SQ_INSTS_SALU', 0) / m['SQ_WAVES']:.4g} SALU, "
                     f"{m.get('SQ_INSTS_LDS', 0) / m['SQ_WAVES']:.4g} LDS, "
                     f"{m.get('SQ_INSTS_VMEM_RD', 0) / m['SQ_WAVES']:.4g} VMEM read, "
                     f"{m.get('SQ_INSTS_VMEM_WR', 0) / m['SQ_WAVES']:.4g} VMEM write instructions")
        if "TCC_HIT" in m and "TCC_MISS" in m:
            L.append(f"- L2 hit rate: TCC_HIT / (TCC_HIT + TCC_MISS) = "
                     f"{m['TCC_HIT'] / (m['TCC_HIT'] + m['TCC_MISS']):.3f}")
    with open(out, "w") as fh:
        fh.write("\n".join(L) + "\n")


def benchline(path, out, command):
    with open(path) as fh:
        line = json.loads([l for l in fh.read().splitlines() if l.startswith("{")][-1])
    h = line["roofline"]
    L = ["# bench.py, every workload (one MI355X)", "", "Command (repository at $R):", "", "```",
         command, "```", "",
         f"Headline `{line['config']['workload']}`: {line['value']:.2f} {line['unit']}, "
         f"{line['ms_per_step']:.4f} ms per step warm, {line['ms_cold_median']:.4f} ms cold median; "
         f"dominant kernel `{h['kernel']}` {h['kernel_ms_mean']:.4f} ms, {h['achieved']:.1f} "
         f"{h['unit']} = {h['frac']:.3f} of {h['peak']:.0f} {h['unit']} ({h['bound']})." , "",
         "| workload | cold median ms | warm ms | dominant kernel ms | dominant achieved | frac | "
         "counter HBM GB/s | eff. TFLOP/s | oracle TFLOP/s (cores) | oracle s, full batch |",
         "|---|---:|---:|---:|---|---:|---:|---:|---:|---:|"]
    for r in line["per_workload"]:
        cb = r.get("cpu_baseline") or {}
        gbs = r.get("counter_hbm_gbs")
        L.append(f"| {r['workload']} | {r['ms_cold_median']:.4f} | {r['ms']:.4f} | "
                 f"{r['dominant_ms_mean']:.4f} | {r['dominant_achieved']:.1f} {r['dominant_unit']} "
                 f"({r['bound']}) | {r['dominant_frac']:.3f} | "
                 f"{'-' if gbs is None else f'{gbs:.0f}'} | {r['effective_tflops']:.2f} | "
                 f"{cb.get('value', float('nan')):.4f} ({cb.get('cores')}) | "
                 f"{cb.get('full_batch_seconds_extrapolated', float('nan')):.2f} |")
    L += ["", "The line:", "", "```json", json.dumps(line), "```"]
    with open(out, "w") as fh:
        fh.write("\n".join(L) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--command", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("out")
    p.add_argument("dirs", nargs="+")
    p.add_argument("--kernel", required=True)
    p.add_argument("--command", required=True)
    b = sub.add_parser("benchline")
    b.add_argument("line")
    b.add_argument("out")
    b.add_argument("--command", required=True)
    a = ap.parse_args()
    if a.mode == "stats":
        stats(a.dir, a.out, a.command)
    elif a.mode == "traffic":
        traffic(a.fetch_dir, a.write_dir, a.copy_mib, a.command)
    elif a.mode == "pmc":
        pmc(a.out, a.kernel, a.command, a.dirs)
    else:
        benchline(a.line, a.out, a.command)


if __name__ == "__main__":
    main()
