"""bench.py's metric formulas against the figures the pages print (tests/golden/)."""
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_metric_examples.txt")


def _rows():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fields, source = line.split("|", 1)
        kind, M, N, K, t_ms, printed, tol = fields.split()
        out.append((kind, int(M), int(N), int(K), float(t_ms), float(printed), float(tol), source.strip()))
    return out


@pytest.mark.parametrize("row", _rows(), ids=lambda r: f"{r[0]}-{r[4]}-{r[5]}")
def test_page_figures(row):
    kind, M, N, K, t_ms, printed, tol, source = row
    if kind == "gflops":
        got = bench.gflops(M, N, K, t_ms)
    else:
        got = bench.flops(M, N, K) / bench.algorithmic_bytes(M, N, K, beta=0.0)
    assert abs(got - printed) <= tol * printed, (got, printed, source)


def test_algorithmic_bytes_counts_c_read_only_with_beta():
    assert bench.algorithmic_bytes(2, 3, 4, 0.0) == 4 * (8 + 12 + 6)
    assert bench.algorithmic_bytes(2, 3, 4, -0.5) == 4 * (8 + 12 + 6) + 4 * 6


def test_metric_string_names_the_workload():
    assert bench.METRIC == "SGEMM GFLOP/s (2MNK/t) at 4096³ FP32 on 1 MI355X; % of FP32 peak"
    assert bench.metric_for(8192, 8192, 8192) == "SGEMM GFLOP/s (2MNK/t) at 8192³ FP32 on 1 MI355X; % of FP32 peak"
    assert "at 1000x1030x999 FP32" in bench.metric_for(1000, 1030, 999)


def test_dpm_table_parsing(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1800Mhz *\n2: 2400Mhz\n")
    assert bench._dpm_levels(str(f)) == (1800, 2400)


def test_bench_refuses_more_than_one_gpu(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_traffic_record_matches_current_kernel_or_is_null():
    """The committed counter summary is used only while the kernel sources are unchanged."""
    import json

    rec = json.load(open(bench.TRAFFIC_FILE))
    value = bench.measured_traffic("sgemm_4096")
    if rec["kernel_source_sha256_16"] == bench.source_digest():
        assert value == rec["fabric_bytes_per_launch"]
    else:
        assert value is None
    assert bench.measured_traffic("sgemm_8192") is None


def test_parity_check_before_timing():
    """bench.parity_check passes the oracle's own result rounded to float32 and fails one
    output moved past the bound (and a NaN), on a small workload checked in full."""
    import numpy as np

    from fp32_gemm_rm_amd.workloads import GemmWorkload, workload_inputs
    from oracle import default_oracle

    w = GemmWorkload("t", 40, 30, 20, 24, 32, 31, "uniform", 7, 1.5, -0.5, "random")
    A, B, C = workload_inputs(w)
    ref, S = default_oracle().full(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc)
    out = C.copy().reshape(w.M, w.ldc)
    out[:, :w.N] = ref.astype(np.float32)
    rec = bench.parity_check(w, A, B, C, out.reshape(-1))
    assert rec["pass"] and rec["outputs_checked"] == w.M * w.N and rec["max_err_over_bound"] < 0.1
    bad = out.copy()
    bad[3, 4] += np.float32(2.0 * (1e-5 * S[3, 4] + 1e-6))
    assert not bench.parity_check(w, A, B, C, bad.reshape(-1))["pass"]
    bad = out.copy()
    bad[5, 6] = np.nan
    assert not bench.parity_check(w, A, B, C, bad.reshape(-1))["pass"]
