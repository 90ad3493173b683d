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


def test_bench_refuses_more_than_one_gpu(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_traffic_record_matches_current_kernel_or_is_null():
    """The committed counter summary is used only while the kernel sources are unchanged."""
    import json

    rec = json.load(open(bench.TRAFFIC_FILE))
    value = bench.measured_traffic("sgemm_4096")
    if rec["kernel_source_sha256_16"] == bench.source_digest():
        assert value == rec["hbm_bytes_per_launch"]
    else:
        assert value is None
    assert bench.measured_traffic("sgemm_8192") is None
