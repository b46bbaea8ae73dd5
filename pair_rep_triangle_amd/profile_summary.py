"""Summarise rocprofv3 CSV output into the short text tables kept under profiles/.

    python -m pair_rep_triangle_amd.profile_summary stats  <kernel_stats.csv>
    python -m pair_rep_triangle_amd.profile_summary traffic <fetch_counter.csv> <write_counter.csv> \
        --copy-mib 256 --workload NAME
    python -m pair_rep_triangle_amd.profile_summary counters <counter.csv> [<counter.csv> ...]
    python -m pair_rep_triangle_amd.profile_summary runs <kernel_trace.csv>

`stats` prints the per-kernel average duration table of a --kernel-trace --stats run.
`traffic` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into bytes per launch,
scaled by what the same counters read for the plain device-to-device copy of
--copy-mib MiB that bench.py runs when given --copy-calibration-mb (the copy kernel
reads and writes exactly that many bytes), and prints one table row per kernel with
the SHA-256 prefix of the kernel sources the counters were taken on.
`counters` prints, per kernel, the mean per dispatch of every counter found in the given
--pmc runs, and the ratios used to read them: MFMA busy per SIMD against the elapsed
GPU clock, instructions per wave, and the share of wave time spent waiting.
`runs` averages, per kernel, the dispatches of a --kernel-trace run that come in runs of
ten or more launches of that kernel alone (bench.py's back-to-back per-kernel regions),
the figure its roofline duration must agree with.
"""

import argparse
import collections
import csv
import hashlib
import os

KERNELS = {"k1_input_gate": "k1_input_gate.hip", "k2_contract": "k2_contract.hip",
           "k3_output_gate_stream": "k3_stream.hip", "k3_output_gate": "k3_output_gate.hip",
           "k0_mask_extents": "k0_mask_extents.hip",
           "pair_transition_wide": "kt_transition_wide.hip", "pair_transition": "kt_transition.hip",
           "ka_project": "ka_attention.hip", "ka_core": "ka_attention.hip"}
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def source_sha(kernel):
    """SHA-256 prefix of the source file of a kernel plus the shared device header."""
    h = hashlib.sha256()
    for f in (KERNELS[kernel], "device_common.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short(name):
    for k in KERNELS:
        if k in name:
            return k
    if "copyBuffer" in name:
        return "copy"
    return None


def stats(path):
    rows = list(csv.DictReader(open(path)))
    print("| kernel | calls | average ns | min ns | max ns |")
    print("|---|---|---|---|---|")
    for r in rows:
        k = short(r["Name"])
        if k and k != "copy":
            print(f"| {k} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")


def counter_means(path, counter):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        k = short(r["Kernel_Name"])
        if k:
            agg[k].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def traffic(fetch_csv, write_csv, copy_mib, workload):
    f = counter_means(fetch_csv, "FETCH_SIZE")
    w = counter_means(write_csv, "WRITE_SIZE")
    want_kib = copy_mib * 1024.0
    fs, ws = want_kib / f["copy"], want_kib / w["copy"]
    print(f"copy calibration ({copy_mib} MiB): FETCH_SIZE {f['copy']:.0f} KiB -> scale {fs:.3f}; "
          f"WRITE_SIZE {w['copy']:.0f} KiB -> scale {ws:.3f}")
    print()
    print("| workload | kernel | source_sha | fetch_bytes | write_bytes | traffic_bytes |")
    print("|---|---|---|---|---|---|")
    for k in KERNELS:
        if k in f and k in w:
            fb, wb = f[k] * fs * 1024, w[k] * ws * 1024
            print(f"| {workload} | {k} | {source_sha(k)} | {fb:.0f} | {wb:.0f} | {fb + wb:.0f} |")


def counters(paths):
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        for r in csv.DictReader(open(path)):
            k = short(r["Kernel_Name"])
            if k and k != "copy":
                agg[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for d in agg.values() for c in d})
    print("| kernel | " + " | ".join(names) + " |")
    print("|---|" + "---|" * len(names))
    for k, d in agg.items():
        cells = [f"{sum(d[c]) / len(d[c]):.4g}" if d.get(c) else "" for c in names]
        print(f"| {k} | " + " | ".join(cells) + " |")
    print()
    # derived: GRBM_GUI_ACTIVE is the elapsed GPU clock summed over the 8 XCDs; the SQ
    # cycle counters are summed over every SIMD (MFMA busy) or wave (wave, wait, busy)
    print("| kernel | MFMA busy per SIMD / elapsed | VALU insts per wave | MFMA insts per wave | "
          "transcendental share of VALU | wait / wave cycles |")
    print("|---|---|---|---|---|---|")
    for k, d in agg.items():
        m = {c: sum(v) / len(v) for c, v in d.items()}
        gui = m.get("GRBM_GUI_ACTIVE")
        waves = m.get("SQ_WAVES")
        row = [k]
        row.append(f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / (gui / 8):.3f}"
                   if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in m else "")
        row.append(f"{m['SQ_INSTS_VALU'] / waves:.0f}" if waves and "SQ_INSTS_VALU" in m else "")
        row.append(f"{m['SQ_INSTS_MFMA'] / waves:.0f}" if waves and "SQ_INSTS_MFMA" in m else "")
        row.append(f"{m['SQ_INSTS_VALU_TRANS_F32'] / m['SQ_INSTS_VALU']:.3f}"
                   if "SQ_INSTS_VALU_TRANS_F32" in m and m.get("SQ_INSTS_VALU") else "")
        row.append(f"{m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.3f}"
                   if "SQ_WAIT_INST_ANY" in m and m.get("SQ_WAVE_CYCLES") else "")
        print("| " + " | ".join(row) + " |")


def runs(path):
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    names = [short(r["Kernel_Name"]) or r["Kernel_Name"][:40] for r in rows]
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    found = collections.defaultdict(list)
    i = 0
    while i < len(rows):
        j = i
        while j < len(rows) and names[j] == names[i]:
            j += 1
        if j - i >= 10:
            found[names[i]].append(dur[i:j])
        i = j
    print("| kernel | runs | dispatches | average us | per-run average us |")
    print("|---|---|---|---|---|")
    for k, rr in found.items():
        allv = [x for r in rr for x in r]
        per = ", ".join(f"{sum(r) / len(r):.2f}" for r in rr)
        print(f"| {k} | {len(rr)} | {len(allv)} | {sum(allv) / len(allv):.2f} | {per} |")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--workload", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    r = sub.add_parser("runs")
    r.add_argument("csv")
    a = ap.parse_args()
    if a.cmd == "stats":
        stats(a.csv)
    elif a.cmd == "runs":
        runs(a.csv)
    elif a.cmd == "counters":
        counters(a.csv)
    else:
        traffic(a.fetch_csv, a.write_csv, a.copy_mib, a.workload)


if __name__ == "__main__":
    main()
