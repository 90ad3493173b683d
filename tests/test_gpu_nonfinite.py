"""NaN and Inf inside the operands: IEEE propagation on the GPU against the oracle.

The oracle evaluates the definition C = alpha*A*B + beta*C in double, where NaN
and Inf propagate by IEEE 754 rules: a NaN in A(i, k) makes row i NaN, an Inf in
B(k, j) makes column j +-Inf where A(i, k) is nonzero and NaN where it is zero
(Inf * 0), and +Inf meeting -Inf in one sum gives NaN.  The pages do not speak to
non-finite values; reading them as IEEE propagation is the plainest one (the
mlqm.cn/news/1180856 troubleshooting table, section 7, lists NaN results as a
failure to hunt down).  Integer inputs in [-4, 4] (zeros included, so Inf * 0
pairs occur) keep every finite output exact, so the comparison is exact:
the same NaN, +Inf and -Inf positions and the same finite values.

The non-finite values sit in the interior, in the last rows of A and columns of
B (the guarded tiles, thin strips and scalar edge tiles of each configuration),
and in the initial C (beta != 0), for every kernel family, every forced MFMA tile
configuration, the default path and the stream-K path.
"""
import numpy as np
import pytest

from fp32_gemm_rm_amd.workloads import C_PAD_SENTINEL, integer_matrix, pad_rows

from .parity import assert_ieee_equal, c_window, check_padding, device

pytestmark = pytest.mark.gpu

FAMILIES = {"naive": 1, "lds_tiled": 2, "regblock": 3, "mfma": 4, "auto": 0}
TILES = {256: 5, 128: 6, 64: 7, 32: 8, 192: 9, 16: 10}
# per forced configuration: shapes with a guarded remainder (>= its partial-tile width)
# along M and a thin one along N, and the reverse; the 256 configuration's thin-strip form
# (both remainders under 16) and its scalar edge tiles (wider remainders); many tile
# columns with a thin right strip (computed inside the tiles in the 64 configuration at
# K >= 640)
SHAPES = {
    256: [(2 * 256 + 4, 256 + 3, 70), (256 + 40, 256 + 33, 45)],
    192: [(2 * 192 + 32, 192 + 5, 70), (192 + 7, 192 + 40, 45), (192 + 20, 48 * 192 + 9, 45)],
    128: [(2 * 128 + 32, 128 + 5, 70), (128 + 7, 128 + 40, 45), (128 + 20, 32 * 128 + 3, 45)],
    64: [(3 * 64 + 20, 64 + 6, 70), (64 + 9, 2 * 64 + 17, 99), (2 * 64 + 20, 16 * 64 + 6, 70),
         (64 + 20, 16 * 64 + 6, 700)],
    32: [(3 * 32 + 6, 2 * 32 + 2, 70), (2 * 32 + 1, 3 * 32 + 5, 45)],
    16: [(3 * 16 + 6, 2 * 16 + 2, 70), (2 * 16 + 1, 3 * 16 + 5, 1045)],
}
FAMILY_SHAPES = [(300, 270, 145), (33, 65, 17)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp32_gemm_rm_amd import load_library

    load_library()


def poisoned_inputs(M, N, K, seed):
    """Integer A, B, C with NaN, +Inf and -Inf planted inside the logical windows."""
    a = integer_matrix(M, K, -4, 4, seed=seed)
    b = integer_matrix(K, N, -4, 4, seed=seed + 1)
    c = integer_matrix(M, N, -4, 4, seed=seed + 2)
    rng = np.random.default_rng(seed)
    ks = rng.integers(0, K, 6)
    # NaN in A: the first row, the middle one and the last one (past the full tiles)
    for i, k in zip((0, M // 2, M - 1), ks[:3]):
        a[i, k] = np.nan
    # +Inf and -Inf in B: column 0, the middle column, and the last one (two opposite Infs)
    b[ks[3], 0] = np.inf
    b[ks[4], N // 2] = -np.inf
    b[ks[3], N - 1] = np.inf
    b[ks[5], N - 1] = -np.inf if ks[5] != ks[3] else np.inf
    # a zero in the column of A that meets the first Inf: Inf * 0 = NaN in that output
    a[1 % M, ks[3]] = 0.0
    # NaN and Inf in the initial C (they reach the output only when beta != 0)
    c[min(1, M - 1), max(N - 2, 0)] = np.nan
    c[max(M - 2, 0), N // 3] = np.inf
    return a, b, c


def run_case(oracle, M, N, K, variant, seed, alpha=-1.5, beta=0.5, ws=None):
    import torch

    from fp32_gemm_rm_amd import sgemm_rm_op_strided_batched_ws

    lda, ldb, ldc = K + 4, N + 4, N + 1
    a, b, c = poisoned_inputs(M, N, K, seed)
    A, B, C = pad_rows(a, lda, np.nan), pad_rows(b, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
    print(f"[nonfinite] {M}x{N}x{K} variant={variant} beta={beta} ws={ws is not None}", flush=True)
    dA, dB, dC = device(A), device(B), device(C)
    s = torch.cuda.current_stream()
    sgemm_rm_op_strided_batched_ws(0, 0, M, N, K, alpha, dA.data_ptr(), lda, 0, dB.data_ptr(), ldb, 0, beta,
                                   dC.data_ptr(), ldc, 0, 1, ws.data_ptr() if ws is not None else None,
                                   ws.numel() if ws is not None else 0, s.cuda_stream, variant)
    s.synchronize()
    out = dC.cpu().numpy()
    ref, _ = oracle.full(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, with_absab=False)
    assert np.isnan(ref).any() and np.isposinf(ref).any() and np.isneginf(ref).any()
    assert_ieee_equal(c_window(out, M, N, ldc), ref, f"{M}x{N}x{K} variant {variant} beta {beta}")
    check_padding(out, C, M, N, ldc)


@pytest.mark.parametrize("beta", [0.5, 0.0])
@pytest.mark.parametrize("variant", list(FAMILIES))
@pytest.mark.parametrize("shape", FAMILY_SHAPES)
def test_families(oracle, variant, shape, beta):
    run_case(oracle, *shape, FAMILIES[variant], seed=sum(shape), beta=beta)


@pytest.mark.parametrize("tiles,shape", [(t, s) for t, shapes in SHAPES.items() for s in shapes])
def test_tile_configurations(oracle, tiles, shape):
    run_case(oracle, *shape, TILES[tiles], seed=tiles + sum(shape))


# 16-byte aligned rows (K and N multiples of 4, so K + 4 and N + 4 too): the LDS-DMA K loops,
# their guarded tiles and thin strips, the packed layout below 256, the 128 configuration's
# two forms, and the 64 one's partial last K-tile and right strip in workgroups of its own
DIRECT_SHAPES = [(256, (256 + 40, 512 + 24, 144)), (256, (512, 256, 64)), (192, (2 * 192 + 32, 192 + 20, 96)),
                 (128, (2 * 128 + 32, 128 + 20, 64)), (128, (2100, 2092, 48)), (64, (3 * 64 + 20, 64 + 8, 96)),
                 (64, (1000, 1032, 68)), (64, (64 + 20, 16 * 64 + 8, 704))]


@pytest.mark.parametrize("tiles,shape", DIRECT_SHAPES)
def test_direct_loops(oracle, tiles, shape):
    run_case(oracle, *shape, TILES[tiles], seed=3 * tiles + sum(shape))


def test_stream_k(oracle):
    """The stream-K path: 20 full 256 x 256 tiles shared by 256 ranges (partial tiles in
    the workspace, added by the fix-up pass), and a shape with one-tile workgroups, stream-K
    tiles and scalar edge tiles around them."""
    import torch

    ws = torch.empty(2 * 256 * 256 * 256 * 4, dtype=torch.uint8, device="cuda")
    run_case(oracle, 1024, 1280, 77, TILES[256], seed=11, ws=ws)
    run_case(oracle, 4352 + 37, 4352 + 19, 40, TILES[256], seed=12, ws=ws)


def test_k_slices(oracle):
    """K slices (the 64 configuration forced, with a workspace): the non-finite values fall in
    different slices of a tile, and the fix-up adds the partial tiles."""
    import torch

    ws = torch.empty(128 << 20, dtype=torch.uint8, device="cuda")
    run_case(oracle, 210, 148, 30000, TILES[64], seed=13, ws=ws)
    run_case(oracle, 64, 64, 100000, TILES[64], seed=14, ws=ws)
