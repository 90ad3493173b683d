"""Summaries of rocprofv3 output for the SGEMM library (kernel traces and counter passes).

One directory per (workload, variant) tag under ``--prof-dir``, as the profiling commands
in the profile summaries create them (``-o run --output-format csv``):

  <tag>/trace/run_kernel_trace.csv, run_kernel_stats.csv   --kernel-trace --stats
  <tag>/sq/run_counter_collection.csv     SQ_INSTS_VALU_FMA_F32 SQ_INSTS_VALU_MFMA_MOPS_F32
                                          SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES
                                          SQ_INSTS_VALU SQ_BUSY_CU_CYCLES SQ_INSTS_LDS SQ_WAVES
                                          GRBM_GUI_ACTIVE
  <tag>/lds/run_counter_collection.csv    SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE
                                          SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR GRBM_GUI_ACTIVE
  <tag>/fetch/run_counter_collection.csv  FETCH_SIZE TCC_EA0_RDREQ_DRAM_sum
  <tag>/write/run_counter_collection.csv  WRITE_SIZE TCC_EA0_WRREQ_DRAM_sum

Counter passes run bench.py with ``--calibrate-copy``: a 256 MiB device copy
(``__amd_rocclr_copyBuffer``) precedes the GEMMs, and each byte or request counter of that
copy against its known size gives the factor that turns the counter into bytes.  FETCH_SIZE
and WRITE_SIZE count traffic between the L2 caches and the memory fabric;
TCC_EA0_RDREQ_DRAM / WRREQ_DRAM count the L2 requests destined for DRAM.  Hits in the
last-level cache in front of HBM are included in both: no counter on this GPU's list
separates them.

Usage (from the repository root):
  python rocprof_summary.py --prof-dir gpurun_out/prof --tag sgemm_4096_auto [--tag ...] \\
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
N_CUS = 256
N_SIMDS = 1024  # 256 CUs x 4 SIMDs
N_XCDS = 8
# nominal shader clock: the MFMA cycles of a SIMD over the traced kernel time at this clock
# are the share of the kernel's duration in which its matrix core is busy (GRBM_GUI_ACTIVE
# under counter collection spans more than the kernel: the passes serialize the dispatches)
CLOCK_MHZ = 2400


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void sgemm_impl::", "")


def kernel_stats(tag_dir: str, last: int):
    """Per library kernel: (name, calls, average us over all calls, average us over the
    last `last` calls (the timed ones), min us)."""
    rows = [r for r in _rows(os.path.join(tag_dir, "trace", "run_kernel_trace.csv"))
            if r["Kernel_Name"].startswith(LIBRARY_PREFIX)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return [(name, len(d), statistics.fmean(d), statistics.fmean(d[-last:]), min(d)) for name, d in by.items()]


def counters(path: str):
    """{dispatch id: (kernel name, {counter: value summed over dimensions})}."""
    out = {}
    for r in _rows(path):
        d = int(r["Dispatch_Id"])
        name, vals = out.setdefault(d, (r["Kernel_Name"], {}))
        vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _library(disp):
    return [v for name, v in disp.values() if name.startswith(LIBRARY_PREFIX)]


def _copy_value(disp, counter):
    vals = [v[counter] for name, v in disp.values() if name == COPY_KERNEL and counter in v]
    if not vals:
        raise SystemExit(f"no {COPY_KERNEL} dispatch with {counter} (run bench.py with --calibrate-copy)")
    return vals[0]


def _mean(lib, counter):
    return statistics.fmean(v[counter] for v in lib)


def summarize(prof_dir: str, tag: str, last: int = 20) -> dict:
    """Figures of one (workload, variant) tag; every counter is a mean over the library's
    dispatches of the pass."""
    import bench
    from fp32_gemm_rm_amd.workloads import WORKLOAD_BY_NAME

    tag_dir = os.path.join(prof_dir, tag)
    workload = next(w for w in sorted(WORKLOAD_BY_NAME, key=len, reverse=True) if tag.startswith(w + "_"))
    w = WORKLOAD_BY_NAME[workload]
    rec = {"tag": tag, "workload": workload, "variant": tag[len(workload) + 1:],
           "kernels": kernel_stats(tag_dir, last), "flops": bench.flops(w.M, w.N, w.K),
           "algorithmic_bytes": bench.algorithmic_bytes(w.M, w.N, w.K, w.beta),
           "algorithmic_reads": 4 * (w.M * w.K + w.K * w.N) + (4 * w.M * w.N if w.beta != 0 else 0),
           "algorithmic_writes": 4 * w.M * w.N}
    path = os.path.join(tag_dir, "fetch", "run_counter_collection.csv")
    if os.path.exists(path):
        disp = counters(path)
        lib = _library(disp)
        f_cal = COPY_BYTES / _copy_value(disp, "FETCH_SIZE")
        d_cal = COPY_BYTES / _copy_value(disp, "TCC_EA0_RDREQ_DRAM_sum")
        rec.update({"fetch_bytes": _mean(lib, "FETCH_SIZE") * f_cal, "fetch_calibration": f_cal / 1024,
                    "dram_read_bytes": _mean(lib, "TCC_EA0_RDREQ_DRAM_sum") * d_cal, "dram_read_calibration": d_cal})
    path = os.path.join(tag_dir, "write", "run_counter_collection.csv")
    if os.path.exists(path):
        disp = counters(path)
        lib = _library(disp)
        w_cal = COPY_BYTES / _copy_value(disp, "WRITE_SIZE")
        d_cal = COPY_BYTES / _copy_value(disp, "TCC_EA0_WRREQ_DRAM_sum")
        rec.update({"write_bytes": _mean(lib, "WRITE_SIZE") * w_cal, "write_calibration": w_cal / 1024,
                    "dram_write_bytes": _mean(lib, "TCC_EA0_WRREQ_DRAM_sum") * d_cal, "dram_write_calibration": d_cal})
    path = os.path.join(tag_dir, "sq", "run_counter_collection.csv")
    if os.path.exists(path):
        lib = _library(counters(path))
        grbm = _mean(lib, "GRBM_GUI_ACTIVE") / N_XCDS  # cycles of the kernel (GRBM counts per XCD)
        rec.update({
            "grbm_cycles": grbm,
            "mfma_busy": _mean(lib, "SQ_VALU_MFMA_BUSY_CYCLES") / (grbm * N_SIMDS),
            "mfma_cycles_per_simd": _mean(lib, "SQ_VALU_MFMA_BUSY_CYCLES") / N_SIMDS,
            # SQ_ACTIVE_INST_VALU counts quad-cycles per SIMD: busy = 4 x count / (SIMDs x cycles)
            "valu_busy": 4 * _mean(lib, "SQ_ACTIVE_INST_VALU") / (grbm * N_SIMDS),
            "valu_fma_flop": _mean(lib, "SQ_INSTS_VALU_FMA_F32") * 64 * 2,
            "mfma_flop": _mean(lib, "SQ_INSTS_VALU_MFMA_MOPS_F32") * 512,
            "valu_insts": _mean(lib, "SQ_INSTS_VALU"), "lds_insts": _mean(lib, "SQ_INSTS_LDS"),
            "waves": _mean(lib, "SQ_WAVES"),
        })
    path = os.path.join(tag_dir, "lds", "run_counter_collection.csv")
    if os.path.exists(path):
        lib = _library(counters(path))
        conf, active = _mean(lib, "SQ_LDS_BANK_CONFLICT"), _mean(lib, "SQ_LDS_IDX_ACTIVE")
        rec.update({"lds_bank_conflict_rate": conf / max(1.0, active - conf),
                    "vmem_rd_insts": _mean(lib, "SQ_INSTS_VMEM_RD"), "vmem_wr_insts": _mean(lib, "SQ_INSTS_VMEM_WR")})
    return rec


def _pct(x):
    return "—" if x is None else f"{100 * x:.1f}%"


def table(recs) -> str:
    """One row per tag: time, rate, pipe busy, FLOP counts, LDS conflicts, memory-side bytes."""
    head = ("| workload | variant | kernel avg (timed calls) us | TFLOP/s | MFMA busy | MFMA cycles / timed us "
            "at 2.4 GHz | VALU busy | "
            "VALU FMA FLOP / 2MNK | MFMA FLOP / 2MNK | LDS conflicts | fabric reads / compulsory | "
            "DRAM-bound reads / compulsory | fabric writes / compulsory |")
    lines = [head, "|" + "---|" * (head.count("|") - 1)]
    for r in recs:
        # one call's kernels (a single kernel, or a main kernel and its fix-up pass)
        t = sum(k[3] for k in r["kernels"]) if r["kernels"] else None
        lines.append("| " + " | ".join([
            r["workload"], r["variant"], f"{t:.1f}" if t else "—",
            f"{r['flops'] / (t * 1e-6) / 1e12:.1f}" if t else "—",
            _pct(r.get("mfma_busy")),
            _pct(r["mfma_cycles_per_simd"] / (t * CLOCK_MHZ)) if t and "mfma_cycles_per_simd" in r else "—",
            _pct(r.get("valu_busy")),
            f"{r['valu_fma_flop'] / r['flops']:.3f}" if "valu_fma_flop" in r else "—",
            f"{r['mfma_flop'] / r['flops']:.3f}" if "mfma_flop" in r else "—",
            f"{100 * r['lds_bank_conflict_rate']:.2f}%" if "lds_bank_conflict_rate" in r else "—",
            f"{r['fetch_bytes'] / r['algorithmic_reads']:.2f}" if "fetch_bytes" in r else "—",
            f"{r['dram_read_bytes'] / r['algorithmic_reads']:.2f}" if "dram_read_bytes" in r else "—",
            f"{r['write_bytes'] / r['algorithmic_writes']:.2f}" if "write_bytes" in r else "—",
        ]) + " |")
    return "\n".join(lines)


def kernels_table(recs) -> str:
    lines = ["| tag | kernel | calls | average us (all) | average us (last timed calls) | min us |",
             "|---|---|---|---|---|---|"]
    for r in recs:
        for name, calls, avg, avg_last, mn in r["kernels"]:
            lines.append(f"| {r['tag']} | `{_short(name)}` | {calls} | {avg:.1f} | {avg_last:.1f} | {mn:.1f} |")
    return "\n".join(lines)


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--prof-dir", required=True)
    p.add_argument("--tag", action="append", required=True, help="<workload>_<variant> directory (repeatable)")
    p.add_argument("--last", type=int, default=20, help="timed calls at the end of each trace")
    p.add_argument("--traffic-json", help="write the per-launch fabric traffic record bench.py reads "
                                          "(from the first tag)")
    p.add_argument("--json", help="write every record as JSON")
    args = p.parse_args(argv)
    recs = [summarize(args.prof_dir, t, args.last) for t in args.tag]
    print(table(recs))
    print()
    print(kernels_table(recs))
    if args.json:
        with open(args.json, "w") as f:
            json.dump(recs, f, indent=1)
    if args.traffic_json:
        import bench

        r = recs[0]
        out = {
            "workload": r["workload"],
            "kernel": [_short(k[0]) for k in r["kernels"]],
            "kernel_source_sha256_16": bench.source_digest(),
            "fabric_bytes_per_launch": round(r["fetch_bytes"] + r["write_bytes"]),
            "fetch_bytes_per_launch": round(r["fetch_bytes"]),
            "write_bytes_per_launch": round(r["write_bytes"]),
            "dram_read_bytes_per_launch": round(r["dram_read_bytes"]),
            "dram_write_bytes_per_launch": round(r["dram_write_bytes"]),
            "fetch_calibration": round(r["fetch_calibration"], 4),
            "write_calibration": round(r["write_calibration"], 4),
            "calibration": f"each counter of a 256 MiB {COPY_KERNEL} in the same process against its size",
            "counters": "FETCH_SIZE and WRITE_SIZE count traffic between the L2 caches and the memory fabric; "
                        "TCC_EA0_RDREQ_DRAM / WRREQ_DRAM the L2 requests destined for DRAM; hits in the "
                        "last-level cache in front of HBM are included in both",
        }
        with open(args.traffic_json, "w") as f:
            json.dump(out, f, indent=1)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
