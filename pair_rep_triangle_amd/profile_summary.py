"""Summarise rocprofv3 CSV output into the short text tables kept under profiles/.

    python -m pair_rep_triangle_amd.profile_summary stats  <kernel_stats.csv>
    python -m pair_rep_triangle_amd.profile_summary traffic <fetch_counter.csv> <write_counter.csv> \
        --copy-mib 256 --workload NAME

`stats` prints the per-kernel average duration table of a --kernel-trace --stats run.
`traffic` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into bytes per launch,
scaled by what the same counters read for the plain device-to-device copy of
--copy-mib MiB that bench.py runs when given --copy-calibration-mb (the copy kernel
reads and writes exactly that many bytes), and prints one table row per kernel with
the SHA-256 prefix of the kernel sources the counters were taken on.
"""

import argparse
import collections
import csv
import hashlib
import os

KERNELS = {"k1_input_gate": "k1_input_gate.hip", "k2_contract": "k2_contract.hip",
           "k3_output_gate": "k3_output_gate.hip", "pair_transition": "kt_transition.hip",
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
    a = ap.parse_args()
    if a.cmd == "stats":
        stats(a.csv)
    else:
        traffic(a.fetch_csv, a.write_csv, a.copy_mib, a.workload)


if __name__ == "__main__":
    main()
