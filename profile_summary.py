"""Summaries of rocprofv3 runs of bench.py, as the markdown tables under
profiles/, and the HBM-traffic record bench.py reads (profiles/hbm_traffic.json).

    python profile_summary.py trace DIR
        kernel table (calls, average / min / max duration, share) of a
        --kernel-trace --stats run
    python profile_summary.py traffic WORKLOAD FETCH_DIR WRITE_DIR [--record]
        bytes read and written per dispatch of the moe_grouped_ffn kernels of
        WORKLOAD (prefill, decode, mxfp4_prefill, mxfp4_decode) from a
        --pmc FETCH_SIZE and a --pmc WRITE_SIZE run of
        `bench.py --calib-copy ...`.  Each counter is scaled by what it reads
        for the 1 GiB device-to-device copy that --calib-copy runs first (the
        process's first copy kernel).  --record stores the per-launch total in
        profiles/hbm_traffic.json with the hash of the kernels' sources.
    python profile_summary.py sq KERNEL_REGEX DIR [DIR ...]
        SQ counters of the matching kernels (average per dispatch) from --pmc
        runs, with MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE /
        8 XCDs x 1024 SIMDs)

Reads only the CSV files rocprofv3 wrote; runs nothing on the GPU.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))

# the kernels of one moe_grouped_ffn call, by workload: (name pattern, which
# dispatches) -- "all" averages every dispatch, "largest"/"smallest" only the
# dispatches with the largest / smallest grid (x quantization runs for every
# call size in the same process)
FFN_KERNELS = {
    "prefill": [(r"ffn_kernel<2, 3, [12], 6, 4, (true|false)>", "all")],
    "decode": [(r"ffn_kernel<2, 3, [12], 1, 4, (true|false)>", "all")],
    "mxfp4_prefill": [(r"ffn_mx_kernel<3, [12], 6, 2>", "all"), (r"x_to_mx_kernel", "largest")],
    "mxfp4_decode": [(r"ffn_mx_kernel<3, [12], 1, 2>", "all"), (r"x_to_mx_kernel", "smallest")],
}


def _csv(d, name):
    hits = glob.glob(os.path.join(d, "**", name), recursive=True)
    if not hits:
        raise SystemExit(f"no {name} under {d}")
    return list(csv.DictReader(open(hits[0])))


def trace(d):
    rows = _csv(d, "*kernel_stats.csv")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    print("| kernel | calls | avg us | min us | max us | share |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        name = re.sub(r"\(.*", "", r["Name"]).replace("void ", "")
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
              f"{100 * float(r['TotalDurationNs']) / total:.1f}% |")


def _counter_rows(d, counter):
    return [r for r in _csv(d, "*counter_collection.csv") if r["Counter_Name"] == counter]


def _calibration(rows):
    """KiB the counter reads for the 1 GiB calibration copy (first copy kernel)."""
    copies = sorted((r for r in rows if "copyBuffer" in r["Kernel_Name"]),
                    key=lambda r: int(r["Dispatch_Id"]))
    if not copies:
        raise SystemExit("no copy kernel: run bench.py with --calib-copy")
    return float(copies[0]["Counter_Value"])


def _per_dispatch(rows, pattern, which):
    sel = [r for r in rows if re.search(pattern, r["Kernel_Name"])]
    if not sel:
        return {}
    if which != "all":
        sizes = [int(r["Grid_Size"]) for r in sel]
        g = max(sizes) if which == "largest" else min(sizes)
        sel = [r for r in sel if int(r["Grid_Size"]) == g]
    by = defaultdict(list)
    for r in sel:
        by[re.sub(r"\(.*", "", r["Kernel_Name"]).replace("void ", "")].append(
            float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in by.items()}


def traffic(workload, fetch_dir, write_dir, record):
    fr, wr = _counter_rows(fetch_dir, "FETCH_SIZE"), _counter_rows(write_dir, "WRITE_SIZE")
    fs, ws = 1048576.0 / _calibration(fr), 1048576.0 / _calibration(wr)
    print(f"calibration: the 1 GiB copy reads FETCH_SIZE = {_calibration(fr):.0f} KiB and "
          f"WRITE_SIZE = {_calibration(wr):.0f} KiB, so bytes = FETCH_SIZE x {fs:.3f} KiB and "
          f"WRITE_SIZE x {ws:.3f} KiB")
    print()
    print("| kernel | read MB | written MB |")
    print("|---|---:|---:|")
    total = 0.0
    for pattern, which in FFN_KERNELS[workload]:
        rd, wt = _per_dispatch(fr, pattern, which), _per_dispatch(wr, pattern, which)
        for k in sorted(rd):
            r_b, w_b = rd[k] * fs * 1024, wt.get(k, 0.0) * ws * 1024
            total += r_b + w_b
            print(f"| `{k}` | {r_b / 1e6:.1f} | {w_b / 1e6:.1f} |")
    print(f"| moe_grouped_ffn total | {total / 1e6:.1f} MB | |")
    if record:
        sys.path.insert(0, ROOT)
        from bench import GEMM_SOURCES, MX_SOURCES, sources_sha
        path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
        rec = json.load(open(path)) if os.path.exists(path) else {}
        mx = workload.startswith("mxfp4")
        # bench.py uses the record only while these sources are unchanged
        rec["mx_src_sha256" if mx else "src_sha256"] = sources_sha(MX_SOURCES if mx else GEMM_SOURCES)
        rec["fetch_scale"], rec["write_scale"] = round(fs, 4), round(ws, 4)
        rec[workload] = {"grouped_ffn_bytes_per_launch": int(round(total))}
        json.dump(rec, open(path, "w"), indent=1)
        print(f"recorded {workload}: {int(round(total))} bytes per launch in {path}")


def sq(pattern, dirs):
    vals = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        for r in _csv(d, "*counter_collection.csv"):
            if re.search(pattern, r["Kernel_Name"]):
                k = re.sub(r"\(.*", "", r["Kernel_Name"]).replace("void ", "")
                vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    for k, cs in vals.items():
        avg = {c: sum(v) / len(v) for c, v in cs.items()}
        print(f"`{k}`")
        for c in sorted(avg):
            print(f"  {c}: {avg[c]:.4g}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
            print(f"  MFMA busy: {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (avg['GRBM_GUI_ACTIVE'] / 8 * 1024):.3f}")
        if "SQ_INSTS_VALU" in avg and "SQ_INSTS_MFMA" in avg:
            print(f"  VALU / MFMA insts: {avg['SQ_INSTS_VALU'] / avg['SQ_INSTS_MFMA']:.2f}")
        for c in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY"):
            if c in avg and "SQ_WAVE_CYCLES" in avg:
                print(f"  {c} / SQ_WAVE_CYCLES: {avg[c] / avg['SQ_WAVE_CYCLES']:.3f}")


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        trace(argv[1])
    elif len(argv) >= 4 and argv[0] == "traffic":
        traffic(argv[1], argv[2], argv[3], "--record" in argv[4:])
    elif len(argv) >= 3 and argv[0] == "sq":
        sq(argv[1], argv[2:])
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
