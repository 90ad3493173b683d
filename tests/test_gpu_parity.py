"""GPU parity: every kernel family against the CPU oracle, through the C ABI.

Every workload (256^3, 1024^3, the ragged 1000 x 1030 x 999 with padded
leading dimensions, 4096^3 and 8192^3) is compared element by element over
all of its outputs, the full-size ones in the launch configuration the
benchmark times.  Closed forms that float32 must reproduce exactly are
compared bit for bit.
"""
import numpy as np
import pytest

from fp32_gemm_rm_amd.workloads import (
    C_PAD_SENTINEL,
    WORKLOAD_BY_NAME,
    integer_matrix,
    make_inputs,
    pad_rows,
    workload_inputs,
)

from .parity import assert_within_bound, c_window, check_padding, device, edge_shapes, run_gemm

pytestmark = pytest.mark.gpu

VARIANTS = {"naive": 1, "lds_tiled": 2, "regblock": 3, "mfma": 4, "auto": 0}
SMALL = ["sgemm_256", "sgemm_1024", "sgemm_ragged_1000x1030x999"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp32_gemm_rm_amd import load_library

    load_library()


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", SMALL)
def test_workload_full(oracle, name, variant):
    w = WORKLOAD_BY_NAME[name]
    print(f"[parity] {name} variant={variant}", flush=True)
    A, B, C = workload_inputs(w)
    out = run_gemm(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, VARIANTS[variant])
    ref, S = oracle.full(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc)
    r = assert_within_bound(c_window(out, w.M, w.N, w.ldc), ref, S, f"{name}/{variant}")
    check_padding(out, C, w.M, w.N, w.ldc)
    print(f"[parity] {name} variant={variant} max err/bound {r:.3g}", flush=True)


@pytest.mark.parametrize("name", ["sgemm_4096", "sgemm_8192"])
def test_workload_full_size(oracle, name):
    """The full-size workloads on the default path, in the call the benchmark times
    (sgemm_rm_ex, variant auto): every one of the M x N outputs against the oracle, within
    the bound, and C's padding (none here) untouched."""
    w = WORKLOAD_BY_NAME[name]
    print(f"[parity] {name} full", flush=True)
    A, B, C = workload_inputs(w)
    out = run_gemm(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, 0)
    print(f"[parity] {name}: GPU done, oracle on {oracle.threads()} threads", flush=True)
    ref, S = oracle.full(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc)
    r = assert_within_bound(c_window(out, w.M, w.N, w.ldc), ref, S, name)
    check_padding(out, C, w.M, w.N, w.ldc)
    print(f"[parity] {name} full: {w.M * w.N} outputs, max err/bound {r:.3g}", flush=True)


@pytest.fixture(scope="module")
def integer_4096(oracle):
    """Integer inputs in [-4, 4] at 4096^3 (C NaN: beta = 0 must not read it) and the
    oracle's full result, shared by the variants below."""
    M = N = K = 4096
    a = integer_matrix(M, K, -4, 4, seed=41)
    b = integer_matrix(K, N, -4, 4, seed=42)
    A, B = a.reshape(-1), b.reshape(-1)
    C = np.full(M * N, np.nan, np.float32)
    ref, _ = oracle.full(M, N, K, 1.0, A, K, B, N, 0.0, C, N, with_absab=False)
    return A, B, C, ref


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_integer_exact_full_size(oracle, integer_4096, variant):
    """Integer inputs make every summation order exact: at 4096^3 every output is
    bit-exact for the MFMA, default and register-blocked paths; the slower families run
    the 1024^3 corner of the same inputs, every output bit-exact."""
    A, B, C, ref = integer_4096
    n = 4096 if variant in ("mfma", "auto", "regblock") else 1024
    print(f"[parity] integer {n}^3 variant={variant}", flush=True)
    # the n x n x n leading corner: A rows of 4096 floats (lda = 4096), B rows likewise
    out = run_gemm(n, n, n, 1.0, A, 4096, B, 4096, 0.0, C[: n * n], n, VARIANTS[variant])
    want = ref if n == 4096 else oracle.full(n, n, n, 1.0, A, 4096, B, 4096, 0.0, None, n, with_absab=False)[0]
    got = out.reshape(n, n).astype(np.float64)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{variant}: {len(bad)} of {n * n} outputs differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_edge_shapes_integer_exact(oracle, variant):
    """Ragged shapes around tile sizes, integer inputs: bit-exact against the oracle,
    with NaN in A/B padding and a sentinel in C padding."""
    for t, (M, N, K) in enumerate(edge_shapes()):
        lda, ldb, ldc = K + (t % 5), N + (t % 3), N + 1 + (t % 4)
        a = integer_matrix(M, K, -4, 4, seed=500 + t)
        b = integer_matrix(K, N, -4, 4, seed=600 + t)
        c = integer_matrix(M, N, -4, 4, seed=700 + t)
        A, B, C = pad_rows(a, lda, np.nan), pad_rows(b, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
        out = run_gemm(M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, VARIANTS[variant])
        ref, _ = oracle.full(M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc)
        got = c_window(out, M, N, ldc).astype(np.float64)
        assert np.array_equal(got, ref), f"shape {(M, N, K)} lds {(lda, ldb, ldc)} variant {variant}"
        check_padding(out, C, M, N, ldc)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_edge_shapes_random_bound(oracle, variant):
    """Ragged random shapes with alpha = 1.5, beta = -0.5 within the bound."""
    for t, (M, N, K) in enumerate(edge_shapes()[::3]):
        lda, ldb, ldc = K + 3, N + 2, N + 1
        A, B, C = make_inputs(M, N, K, lda, ldb, ldc, "normal", seed=800 + t, c_init="random")
        out = run_gemm(M, N, K, 1.5, A, lda, B, ldb, -0.5, C, ldc, VARIANTS[variant])
        ref, S = oracle.full(M, N, K, 1.5, A, lda, B, ldb, -0.5, C, ldc)
        assert_within_bound(c_window(out, M, N, ldc), ref, S, f"{(M, N, K)}/{variant}")
        check_padding(out, C, M, N, ldc)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_closed_forms(variant):
    v = VARIANTS[variant]
    # identity: A = I gives C = B bit for bit
    M = K = 192
    N = 200
    eye = pad_rows(np.eye(M, K, dtype=np.float32), K + 4, np.nan)
    _, B, C = make_inputs(M, N, K, K + 4, N + 4, N + 4, "normal", seed=9, c_init="nan")
    out = run_gemm(M, N, K, 1.0, eye, K + 4, B, N + 4, 0.0, C, N + 4, v)
    np.testing.assert_array_equal(c_window(out, M, N, N + 4), B.reshape(K, N + 4)[:, :N])
    # all ones: C = K exactly, and 1.5K - 0.5 with beta = -0.5, C = 1
    M, N, K = 130, 250, 777
    ones_a = np.ones(M * K, np.float32)
    ones_b = np.ones(K * N, np.float32)
    out = run_gemm(M, N, K, 1.0, ones_a, K, ones_b, N, 0.0, np.full(M * N, np.nan, np.float32), N, v)
    np.testing.assert_array_equal(out.reshape(M, N), np.full((M, N), K, np.float32))
    out = run_gemm(M, N, K, 1.5, ones_a, K, ones_b, N, -0.5, np.ones(M * N, np.float32), N, v)
    np.testing.assert_array_equal(out.reshape(M, N), np.full((M, N), 1.5 * K - 0.5, np.float32))
    # rank one: K = 1 gives fl(a_i * b_j) bit for bit
    M, N, K = 300, 257, 1
    A, B, C = make_inputs(M, N, K, 1, N, N, "normal", seed=10, c_init="nan")
    out = run_gemm(M, N, K, 1.0, A, 1, B, N, 0.0, C, N, v)
    np.testing.assert_array_equal(out.reshape(M, N), np.outer(A[:M], B[:N]).astype(np.float32))


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_alpha_zero_and_k_zero(variant):
    """alpha = 0 (or K = 0) gives beta*C bit for bit and never reads A or B (NaN)."""
    M, N, K = 100, 70, 33
    A = np.full(M * K, np.nan, np.float32)
    B = np.full(K * N, np.nan, np.float32)
    _, _, C = make_inputs(M, N, K, K, N, N + 5, "uniform", seed=14, c_init="random")
    out = run_gemm(M, N, K, 0.0, A, K, B, N, -0.5, C, N + 5, VARIANTS[variant])
    want = (np.float32(-0.5) * c_window(C, M, N, N + 5)).astype(np.float32)
    np.testing.assert_array_equal(c_window(out, M, N, N + 5), want)
    check_padding(out, C, M, N, N + 5)
    out = run_gemm(M, N, 0, 1.0, A, 1, B, N, 0.0, C, N + 5, VARIANTS[variant])
    np.testing.assert_array_equal(c_window(out, M, N, N + 5), np.zeros((M, N), np.float32))
    out = run_gemm(M, N, 0, 1.0, A, 1, B, N, 1.0, C, N + 5, VARIANTS[variant])
    np.testing.assert_array_equal(out, C)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_beta_zero_ignores_nan_c(oracle, variant):
    M, N, K = 257, 129, 65
    A, B, C = make_inputs(M, N, K, K, N, N, "uniform", seed=15, c_init="nan")
    out = run_gemm(M, N, K, 1.0, A, K, B, N, 0.0, C, N, VARIANTS[variant])
    ref, S = oracle.full(M, N, K, 1.0, A, K, B, N, 0.0, C, N)
    assert_within_bound(out.reshape(M, N), ref, S, f"beta0/{variant}")


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_misaligned_pointers(oracle, variant):
    """Base pointers off 16-byte alignment and odd leading dimensions take the scalar-load path."""
    import torch

    M, N, K = 300, 270, 145
    lda, ldb, ldc = K + 1, N + 3, N + 1
    A, B, C = make_inputs(M, N, K, lda, ldb, ldc, "uniform", seed=16, c_init="random")
    dA = device(np.concatenate([np.zeros(1, np.float32), A]))
    dB = device(np.concatenate([np.zeros(3, np.float32), B]))
    dC = device(np.concatenate([np.zeros(2, np.float32), C]))
    from fp32_gemm_rm_amd import sgemm_rm_ex

    s = torch.cuda.current_stream()
    sgemm_rm_ex(M, N, K, 1.5, dA.data_ptr() + 4, lda, dB.data_ptr() + 12, ldb, -0.5, dC.data_ptr() + 8, ldc,
                s.cuda_stream, VARIANTS[variant])
    s.synchronize()
    out = dC.cpu().numpy()[2:]
    ref, S = oracle.full(M, N, K, 1.5, A, lda, B, ldb, -0.5, C, ldc)
    assert_within_bound(c_window(out, M, N, ldc), ref, S, f"misaligned/{variant}")
    check_padding(out, C, M, N, ldc)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_deterministic(variant):
    w = WORKLOAD_BY_NAME["sgemm_ragged_1000x1030x999"]
    A, B, C = workload_inputs(w)
    o1 = run_gemm(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, VARIANTS[variant])
    o2 = run_gemm(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, VARIANTS[variant])
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


def test_side_stream_ordering(oracle):
    """Work enqueued on a non-default stream sees the producer's writes and is ordered after them."""
    import torch

    w = WORKLOAD_BY_NAME["sgemm_1024"]
    A, B, C = workload_inputs(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dA, dB, dC = device(A), device(B), device(C)
        dC.fill_(np.nan)  # beta == 0: must be ignored
        from fp32_gemm_rm_amd import sgemm

        sgemm(dA.view(w.M, w.K), dB.view(w.K, w.N), dC.view(w.M, w.N), 1.0, 0.0)
    s.synchronize()
    ref, S = oracle.full(w.M, w.N, w.K, 1.0, A, w.K, B, w.N, 0.0, C, w.N)
    assert_within_bound(dC.cpu().numpy().reshape(w.M, w.N), ref, S, "side stream")


def test_invalid_arguments_on_device():
    from fp32_gemm_rm_amd import SgemmError, sgemm_rm_ex

    with pytest.raises(SgemmError) as e:
        sgemm_rm_ex(4, 4, 4, 1.0, 0, 4, 0, 4, 0.0, 0, 4, 0, 4)
    assert e.value.code == -5


def test_single_hip_runtime():
    """torch and the library share one HIP runtime in the process."""
    import torch  # noqa: F401

    from fp32_gemm_rm_amd import load_library

    load_library()
    maps = open("/proc/self/maps").read().splitlines()
    libs = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(libs) == 1, libs


# Shapes per MFMA tile configuration (forced through its variant): full tiles only,
# and full tiles plus partial ones (scalar edge tiles, or guarded MFMA tiles for 32).
TILE_SHAPES = {
    256: [(4096, 4096, 17), (4000, 3900, 77)],
    192: [(3072, 3072, 300), (2000, 1950, 129)],
    128: [(2048, 2048, 300), (2176, 2048, 300), (2000, 1950, 129)],  # one layer, 272 tiles, guarded one layer
    64: [(1024, 1024, 129), (1000, 990, 129)],
    32: [(512, 512, 300), (1000, 1030, 99)],
    16: [(256, 256, 300), (100, 90, 129)],
}


@pytest.mark.parametrize("tiles,M,N,K", [(t, *s) for t, shapes in TILE_SHAPES.items() for s in shapes])
def test_tile_configs_integer_exact(oracle, tiles, M, N, K):
    """Every MFMA tile configuration, with and without partial tiles: bit-exact on integer
    inputs, padded leading dimensions, NaN padding in A/B, sentinel in C.  The default
    path runs on the same inputs too."""
    from fp32_gemm_rm_amd import TILE_VARIANTS

    lda, ldb, ldc = K + 4, N + 8, N + 3
    a = integer_matrix(M, K, -4, 4, seed=M + K)
    b = integer_matrix(K, N, -4, 4, seed=N + K)
    c = integer_matrix(M, N, -4, 4, seed=M + N)
    A, B, C = pad_rows(a, lda, np.nan), pad_rows(b, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
    ref, _ = oracle.full(M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc)
    for variant in (TILE_VARIANTS[tiles], VARIANTS["auto"]):
        out = run_gemm(M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, variant)
        got = c_window(out, M, N, ldc).astype(np.float64)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"variant {variant}: {len(bad)} mismatches, first at {bad[:3].tolist()}"
        check_padding(out, C, M, N, ldc)


# Partial tiles: a remainder of 16 or more rows (columns; 4 in the 32 configuration) runs as
# guarded MFMA tiles (guarded along M only, along N only, or both: separate code paths), a
# thinner one as thin strips; so do the last 1-3 columns of B (rows of A^T) when the guarded
# remainder is not a multiple of 4.  Shapes put remainders on both sides of 16, in
# either dimension, and cover matrices smaller than one tile or thinner than 16; the
# long-K cases give every wavefront of a thin strip 64 or more MFMA steps (its long-slice
# form).
PARTIAL_SHAPES = {
    # 256: remainders thinner than 16 run as thin strips after the full tiles, wider ones as
    # scalar edge tiles (TILE_SHAPES)
    256: [(2 * 256 + 4, 256 + 3, 70), (256 + 15, 2 * 256, 45), (2 * 256, 256 + 1, 33), (12, 9, 40),
          (256 + 7, 256 + 12, 1100)],
    192: [(2 * 192 + 32, 192 + 31, 70), (192 + 15, 2 * 192 + 16, 45), (3 * 192 + 5, 192 + 3, 1100), (100, 300, 70),
          (12, 300, 45)],
    128: [(3 * 128 + 32, 2 * 128 + 31, 70), (3 * 128 + 31, 2 * 128 + 32, 70), (128 + 16, 128 + 15, 70),
          (128 + 15, 128 + 16, 33), (2 * 128 + 7, 3 * 128 + 1, 70), (100, 300, 70), (20, 300, 45), (300, 20, 45),
          (12, 300, 45), (300, 12, 45), (9, 7, 45), (2 * 128 + 5, 128 + 3, 1100),
          (2100, 2090, 77)],  # 289 guarded tiles: the two-workgroup form (smaller grids: 4 x 2 wavefronts)
    32: [(3 * 32 + 2, 2 * 32 + 3, 70), (3 * 32 + 5, 2 * 32 + 7, 45), (1, 40, 33), (40, 1, 33), (3, 3, 5),
         (2 * 32 + 6, 3 * 32 + 6, 300)],
    64: [(5 * 64 + 16, 4 * 64 + 15, 70), (5 * 64 + 15, 4 * 64 + 16, 70), (64 + 15, 64 + 15, 70),
         (1000, 1030, 99), (40, 200, 45), (10, 200, 45), (200, 10, 45), (1, 1, 300), (3 * 64 + 1, 2 * 64 + 14, 1),
         (64 + 3, 2 * 64 + 9, 2100)],
    # 16: every block guarded where M or N is not a multiple of 16; K below one group, K
    # slices of every length (long ones take the 4-group chunks), and the K tail
    16: [(17, 33, 70), (1, 1, 5), (15, 300, 45), (300, 7, 1100), (5 * 16 + 3, 3 * 16 + 9, 4100)],
}


@pytest.mark.parametrize("tiles,M,N,K", [(t, *s) for t, shapes in PARTIAL_SHAPES.items() for s in shapes])
def test_partial_tile_forms_integer_exact(oracle, tiles, M, N, K):
    """Full and guarded MFMA tiles side by side (forced tile configuration): bit-exact on
    integer inputs, NaN padding in A/B, sentinel in C."""
    from fp32_gemm_rm_amd import TILE_VARIANTS

    lda, ldb, ldc = K + 4, N + 4, N + 1
    a = integer_matrix(M, K, -4, 4, seed=M + 2 * K)
    b = integer_matrix(K, N, -4, 4, seed=N + 2 * K)
    c = integer_matrix(M, N, -4, 4, seed=M + 2 * N)
    A, B, C = pad_rows(a, lda, np.nan), pad_rows(b, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
    ref, _ = oracle.full(M, N, K, -1.5, A, lda, B, ldb, 0.5, C, ldc)
    out = run_gemm(M, N, K, -1.5, A, lda, B, ldb, 0.5, C, ldc, TILE_VARIANTS[tiles])
    got = c_window(out, M, N, ldc).astype(np.float64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"tiles {tiles} {M}x{N}x{K}: {len(bad)} mismatches, first at {bad[:3].tolist()}"
    check_padding(out, C, M, N, ldc)


# Right thin strips computed inside the MFMA tiles (operands stored row-major, the 64
# configuration, at least 16 tile columns, K >= 640): tile (bm, bn) takes 4 rows of the
# strip.  Shapes: strips 1-15 wide past full tiles, the last 1-3 columns of a guarded
# remainder, guarded tile rows (strip rows past the last tile's), M below one tile, K
# tails, even and odd K-tile counts, and the smallest tile-column count that fuses; K
# just under the threshold keeps the strip in workgroups of its own, as do the 192 and
# 128 configurations' shapes with as many tile columns.
FUSED_SHAPES = {
    64: [(5 * 64 + 20, 16 * 64 + 11, 999), (5 * 64, 16 * 64 + 18, 640), (17, 16 * 64 + 1, 673),
         (2 * 64 + 30, 40 * 64 + 15, 2100), (64, 16 * 64 + 9, 1024 + 32), (1000, 1030, 999),
         (3 * 64 + 5, 16 * 64 + 3, 639), (2 * 64, 16 * 64 + 7, 70)],
    192: [(2 * 192 + 40, 48 * 192 + 7, 70), (192 + 17, 48 * 192 + 16 + 3, 33)],
    128: [(300, 32 * 128 + 5, 77), (20, 32 * 128 + 15, 45), (3 * 128, 33 * 128 + 1, 16 * 9 + 5)],
}


@pytest.mark.parametrize("tiles,M,N,K", [(t, *s) for t, shapes in FUSED_SHAPES.items() for s in shapes])
def test_fused_right_strip_integer_exact(oracle, tiles, M, N, K):
    """Right strips inside the tiles: bit-exact on integer inputs (padded leading
    dimensions, NaN padding in A/B, sentinel in C), with beta != 0 and with beta = 0 over
    a NaN C (which must not reach the output); the default path on the same inputs."""
    from fp32_gemm_rm_amd import TILE_VARIANTS

    lda, ldb, ldc = K + 4, N + 4, N + 1
    a = integer_matrix(M, K, -4, 4, seed=M + 3 * K)
    b = integer_matrix(K, N, -4, 4, seed=N + 3 * K)
    c = integer_matrix(M, N, -4, 4, seed=M + 3 * N)
    A, B, C = pad_rows(a, lda, np.nan), pad_rows(b, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
    print(f"[parity] fused strip tiles {tiles} {M}x{N}x{K}", flush=True)
    ref, _ = oracle.full(M, N, K, -1.5, A, lda, B, ldb, 0.5, C, ldc)
    for variant in (TILE_VARIANTS[tiles], VARIANTS["auto"]):
        out = run_gemm(M, N, K, -1.5, A, lda, B, ldb, 0.5, C, ldc, variant)
        got = c_window(out, M, N, ldc).astype(np.float64)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"variant {variant}: {len(bad)} mismatches, first at {bad[:3].tolist()}"
        check_padding(out, C, M, N, ldc)
    Cn = C.copy()
    Cn.reshape(M, ldc)[:, :N] = np.nan
    ref0, _ = oracle.full(M, N, K, 2.0, A, lda, B, ldb, 0.0, Cn, ldc)
    out = run_gemm(M, N, K, 2.0, A, lda, B, ldb, 0.0, Cn, ldc, TILE_VARIANTS[tiles])
    got = c_window(out, M, N, ldc).astype(np.float64)
    bad = np.argwhere(got != ref0)
    assert bad.size == 0, f"beta 0: {len(bad)} mismatches, first at {bad[:3].tolist()}"
    check_padding(out, Cn, M, N, ldc)


@pytest.mark.parametrize("tiles", [256, 192, 128, 64, 32, 16])
def test_tile_configs_random_bound(oracle, tiles):
    """Each forced tile configuration on the ragged 1000 x 1030 x 999 workload (alpha 1.5,
    beta -0.5, padded leading dimensions), within the bound."""
    from fp32_gemm_rm_amd import TILE_VARIANTS

    w = WORKLOAD_BY_NAME["sgemm_ragged_1000x1030x999"]
    A, B, C = workload_inputs(w)
    out = run_gemm(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc, TILE_VARIANTS[tiles])
    ref, S = oracle.full(w.M, w.N, w.K, w.alpha, A, w.lda, B, w.ldb, w.beta, C, w.ldc)
    assert_within_bound(c_window(out, w.M, w.N, w.ldc), ref, S, f"tiles {tiles}")
    check_padding(out, C, w.M, w.N, w.ldc)


@pytest.mark.parametrize("variant,N", [("mfma", 64), ("auto", 64), ("regblock", 64), ("lds_tiled", 64), ("naive", 4)])
def test_offsets_past_2_pow_31(oracle, variant, N):
    """A with more than 2^31 elements (65539 x 32772): row offsets i*lda need 64 bits.
    A lives only on the device (integer pattern drawn there); the oracle gets the sampled
    rows of A, so every check is bit-exact on integer inputs."""
    import torch

    M, K = 65539, 32768
    lda, ldb, ldc = K + 4, N, N
    assert M * lda > 2**31
    gen = torch.Generator(device="cuda").manual_seed(77)
    dA = torch.randint(-2, 3, (M * lda,), generator=gen, device="cuda", dtype=torch.int8).to(torch.float32)
    b = integer_matrix(K, N, -2, 2, seed=78)
    dB = device(b.reshape(-1))
    dC = torch.full((M * ldc,), float("nan"), device="cuda")
    out = run_gemm(M, N, K, 1.0, None, lda, None, ldb, 0.0, None, ldc, VARIANTS[variant], tensors=(dA, dB, dC))
    rows = np.array([0, 1, 32767, 32768, 65535, 65536, 65537, 65538])
    a_rows = dA.view(M, lda)[torch.from_numpy(rows).cuda()].cpu().numpy().reshape(-1)
    r = np.repeat(np.arange(len(rows)), N)
    c = np.tile(np.arange(N), len(rows))
    ref, _ = oracle.entries(len(rows), N, K, 1.0, a_rows, lda, b.reshape(-1), ldb, 0.0, None, ldc, r, c)
    got = out.reshape(M, ldc)[rows][:, :N].reshape(-1).astype(np.float64)
    np.testing.assert_array_equal(got, ref)
    del dA
    torch.cuda.empty_cache()


# K-tile depth of each tile configuration (the K loop runs a steady state over pairs of
# full K-tiles and a general tail; these K values put its boundaries in every place).
TILE_BK = {256: 16, 192: 16, 128: 16, 64: 32, 32: 64, 16: 16}


@pytest.mark.parametrize(
    "tiles,M,N,bk",
    [(t, t + 40, t + 24, TILE_BK[t]) for t in (256, 192, 128, 64, 32, 16)]
    # the 256 configuration's thin-strip form
    + [(256, 2 * 256 + 5, 256 + 3, 16)]
    # exact 128 x 128 tiles, at most one per CU: the one-layer form (4 x 2 wavefronts)
    + [(128, 256, 384, 16)],
)
def test_k_loop_boundaries_integer_exact(oracle, tiles, M, N, bk):
    """K from 1 to nine K-tiles (full, ragged, odd and even tile counts) for each forced
    tile configuration, on a shape with full and partial tiles (and on full tiles only for
    the one-layer form of the 128 configuration): bit-exact."""
    from fp32_gemm_rm_amd import TILE_VARIANTS

    for K in sorted({1, 3, bk - 1, bk, bk + 1, 2 * bk, 2 * bk + 5, 3 * bk - 1, 3 * bk, 4 * bk, 4 * bk + 1,
                     5 * bk, 5 * bk + 7, 6 * bk, 7 * bk + 3, 8 * bk, 9 * bk - 2}):
        lda, ldb, ldc = K + 3, N + 5, N + 2
        a = integer_matrix(M, K, -4, 4, seed=3 * K + 1)
        b = integer_matrix(K, N, -4, 4, seed=3 * K + 2)
        c = integer_matrix(M, N, -4, 4, seed=3 * K + 3)
        A, B, C = pad_rows(a, lda, np.nan), pad_rows(b, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
        out = run_gemm(M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, TILE_VARIANTS[tiles])
        ref, _ = oracle.full(M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc)
        got = c_window(out, M, N, ldc).astype(np.float64)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"tiles {tiles} K {K}: {len(bad)} mismatches, first at {bad[:3].tolist()}"
        check_padding(out, C, M, N, ldc)
