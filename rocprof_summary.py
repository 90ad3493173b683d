"""Summaries of rocprofv3 output for the SGEMM library (kernel traces and counter passes).

Reads the CSV files that ``rocprofv3 --kernel-trace --stats`` and ``rocprofv3 --pmc``
write (``-o run --output-format csv``) and prints the figures the profile summaries
quote; with ``--traffic-json`` it also writes the per-launch fabric traffic record that
``bench.py`` reports as ``roofline.traffic``.

Layout under ``--prof-dir`` (one directory per run, as bench.py's profiling commands
create them):
  trace_<workload>/run_kernel_stats.csv
  pmc_<workload>_FETCH_SIZE/run_counter_collection.csv
  pmc_<workload>_WRITE_SIZE/run_counter_collection.csv
  pmc_<workload>_SQ_LDS_BANK_CONFLICT/run_counter_collection.csv   (the SQ / GRBM pass)

Counter passes run bench.py with ``--calibrate-copy``: a 256 MiB device copy
(``__amd_rocclr_copyBuffer``) precedes the GEMMs, and FETCH_SIZE / WRITE_SIZE of that copy
against its known size give the factor that turns each counter into bytes.

Usage (from the repository root):
  python rocprof_summary.py --prof-dir gpurun_out/prof --workload sgemm_4096 \\
      [--traffic-json profiles/traffic_mfma_sgemm_4096.json]
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 256 << 20
LIBRARY_PREFIX = "void sgemm_impl::"
N_SIMDS = 1024  # 256 CUs x 4 SIMDs
N_XCDS = 8


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def kernel_stats(prof_dir: str, workload: str):
    """(name, calls, average us, min us, max us) of the library's kernels in the trace."""
    out = []
    for r in _rows(os.path.join(prof_dir, f"trace_{workload}", "run_kernel_stats.csv")):
        if r["Name"].startswith(LIBRARY_PREFIX):
            out.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                        float(r["MaxNs"]) / 1e3))
    return out


def counters(path: str):
    """{dispatch id: (kernel name, {counter: value summed over dimensions})}."""
    out = {}
    for r in _rows(path):
        d = int(r["Dispatch_Id"])
        name, vals = out.setdefault(d, (r["Kernel_Name"], {}))
        vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _library_mean(disp, counter):
    vals = [v[counter] for name, v in disp.values() if name.startswith(LIBRARY_PREFIX)]
    return statistics.fmean(vals), len(vals)


def _calibration(disp, counter):
    """Bytes per counter unit, from the 256 MiB copy: the counter is in KiB per dispatch."""
    vals = [v[counter] for name, v in disp.values() if name == COPY_KERNEL]
    if not vals:
        raise SystemExit(f"no {COPY_KERNEL} dispatch in the {counter} pass (run bench.py with --calibrate-copy)")
    return COPY_BYTES / vals[0]


def summarize(prof_dir: str, workload: str) -> dict:
    import bench
    from fp32_gemm_rm_amd.workloads import WORKLOAD_BY_NAME

    w = WORKLOAD_BY_NAME[workload]
    rec = {"workload": workload, "kernels": kernel_stats(prof_dir, workload)}
    fetch = counters(os.path.join(prof_dir, f"pmc_{workload}_FETCH_SIZE", "run_counter_collection.csv"))
    write = counters(os.path.join(prof_dir, f"pmc_{workload}_WRITE_SIZE", "run_counter_collection.csv"))
    f_cal, w_cal = _calibration(fetch, "FETCH_SIZE"), _calibration(write, "WRITE_SIZE")
    f_mean, n_f = _library_mean(fetch, "FETCH_SIZE")
    w_mean, n_w = _library_mean(write, "WRITE_SIZE")
    rec.update({
        "fetch_bytes_per_launch": f_mean * f_cal, "write_bytes_per_launch": w_mean * w_cal,
        "fetch_calibration": f_cal / 1024, "write_calibration": w_cal / 1024, "dispatches": min(n_f, n_w),
        "algorithmic_bytes": bench.algorithmic_bytes(w.M, w.N, w.K, w.beta),
        "algorithmic_reads": 4 * (w.M * w.K + w.K * w.N) + (4 * w.M * w.N if w.beta != 0 else 0),
        "algorithmic_writes": 4 * w.M * w.N, "flops": bench.flops(w.M, w.N, w.K),
    })
    sq_path = os.path.join(prof_dir, f"pmc_{workload}_SQ_LDS_BANK_CONFLICT", "run_counter_collection.csv")
    if os.path.exists(sq_path):
        sq = counters(sq_path)
        lib = [v for name, v in sq.values() if name.startswith(LIBRARY_PREFIX)]

        def mean(c):
            return statistics.fmean(v[c] for v in lib)

        grbm_per_xcd = mean("GRBM_GUI_ACTIVE") / N_XCDS
        rec.update({
            "mfma_busy": mean("SQ_VALU_MFMA_BUSY_CYCLES") / (grbm_per_xcd * N_SIMDS),
            "lds_bank_conflict_rate": mean("SQ_LDS_BANK_CONFLICT") /
            max(1.0, mean("SQ_LDS_IDX_ACTIVE") - mean("SQ_LDS_BANK_CONFLICT")),
            "mfma_flop": mean("SQ_INSTS_VALU_MFMA_MOPS_F32") * 512,
            "grbm_gui_active_per_xcd": grbm_per_xcd,
        })
    return rec


def markdown(rec: dict) -> str:
    lines = ["| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for name, calls, avg, mn, mx in rec["kernels"]:
        short = name.split("(")[0].replace("void sgemm_impl::", "")
        lines.append(f"| `{short}` | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} |")
    lines += ["", "| quantity (per launch) | value |", "|---|---|",
              f"| FETCH_SIZE x {rec['fetch_calibration']:.4f} KiB | {rec['fetch_bytes_per_launch'] / 1e6:.1f} MB |",
              f"| WRITE_SIZE x {rec['write_calibration']:.4f} KiB | {rec['write_bytes_per_launch'] / 1e6:.1f} MB |",
              f"| algorithmic bytes (reads, writes) | {rec['algorithmic_bytes'] / 1e6:.1f} MB "
              f"({rec['algorithmic_reads'] / 1e6:.1f}, {rec['algorithmic_writes'] / 1e6:.1f}) |",
              f"| measured / algorithmic | {(rec['fetch_bytes_per_launch'] + rec['write_bytes_per_launch']) / rec['algorithmic_bytes']:.2f} |"]
    if "mfma_busy" in rec:
        lines += [f"| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs)) | "
                  f"{100 * rec['mfma_busy']:.1f}% |",
                  f"| LDS bank conflicts (SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT)) | "
                  f"{100 * rec['lds_bank_conflict_rate']:.2f}% |",
                  f"| SQ_INSTS_VALU_MFMA_MOPS_F32 x 512 | {rec['mfma_flop']:.4g} FLOP (2MNK = {rec['flops']:.4g}) |",
                  f"| GRBM_GUI_ACTIVE per XCD | {rec['grbm_gui_active_per_xcd'] / 1e6:.3f} M cycles |"]
    return "\n".join(lines)


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--prof-dir", required=True)
    p.add_argument("--workload", required=True)
    p.add_argument("--traffic-json", help="write the per-launch traffic record bench.py reads")
    args = p.parse_args(argv)
    rec = summarize(args.prof_dir, args.workload)
    print(markdown(rec))
    if args.traffic_json:
        import bench

        kernels = [k[0].split("(")[0].replace("void ", "") for k in rec["kernels"]]
        out = {
            "workload": args.workload,
            "kernel": kernels[0] if len(kernels) == 1 else kernels,
            "kernel_source_sha256_16": bench.source_digest(),
            "fabric_bytes_per_launch": round(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]),
            "fetch_bytes_per_launch": round(rec["fetch_bytes_per_launch"]),
            "write_bytes_per_launch": round(rec["write_bytes_per_launch"]),
            "fetch_calibration": round(rec["fetch_calibration"], 4),
            "write_calibration": round(rec["write_calibration"], 4),
            "calibration": f"FETCH_SIZE and WRITE_SIZE of a 256 MiB {COPY_KERNEL} in the same process",
            "counters": "FETCH_SIZE and WRITE_SIZE count traffic between the L2 caches and the memory fabric; "
                        "hits in the last-level cache in front of HBM are included",
            "dispatches": rec["dispatches"],
        }
        with open(args.traffic_json, "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
