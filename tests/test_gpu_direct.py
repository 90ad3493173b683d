"""The two K loops of the 256, 192, 128 and 64 configurations: LDS-DMA loads and
register-staged loads.

Where every row of A and B is 16-byte aligned, K is a multiple of 16 and the byte offsets
inside a K-tile fit in 31 bits, the 256 x 256 tiles load their operands straight into LDS
(buffer_load ... lds, on 4 x 2 wavefronts); a leading dimension past about 2.1 million
floats (along k), or a K tail, takes the register-staged pipeline (2 x 2 wavefronts)
instead.  Both must give the oracle's result bit for bit on integer inputs (every partial
sum is exact), and, since both read the same LDS layout and add each output's products in
the same order, the same bits as each other on random inputs too.  Shapes cover fewer
K-tiles than LDS stages, B stored transposed, and a K tail (both runs then staged).  The
operand padding is NaN, so a read past a row reaches C.  The direct loop also runs the tiles
that reach past M or N (guarded tiles, with thin strips for remainders under 16).  The 192,
128 and 64 configurations take the direct loop under the same conditions (the 64 one loads a
partial last K-tile through registers), their operands stored along m or n in a packed,
XOR-swizzled LDS layout; there the register-staged loop runs for rows that are not 16-byte
aligned.
"""
import numpy as np
import pytest

from fp32_gemm_rm_amd.workloads import integer_matrix

from .parity import c_window

pytestmark = pytest.mark.gpu

T256 = 5  # SGEMM_RM_VARIANT_MFMA_T256
T128 = 6  # SGEMM_RM_VARIANT_MFMA_T128
T192 = 9  # SGEMM_RM_VARIANT_MFMA_T192
T64 = 7  # SGEMM_RM_VARIANT_MFMA_T64
# smallest multiple of 4 with 255 * ld * 4 bytes >= 2^31: rows along k this far apart leave
# the direct pipeline
HUGE_LD = ((2**31 + 4 * 255 - 1) // (4 * 255) + 3) // 4 * 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp32_gemm_rm_amd import load_library

    load_library()
    yield
    torch.cuda.empty_cache()


def _ld4(n):
    return (n + 3) // 4 * 4


def _stored_on_device(x, ld):
    """Row-major rows x cols matrix x on the device with leading dimension ld, NaN padding."""
    import torch

    rows, cols = x.shape
    buf = torch.full((rows * ld,), float("nan"), device="cuda")
    buf.view(rows, ld)[:, :cols] = torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    return buf


def _run(M, N, K, a, lda, b, ldb, tb, c, alpha, beta, ta=0, variant=T256):
    """C := alpha op(A) op(B) + beta C on a forced configuration (256 by default); a is op(A)
    (M x K), stored transposed (K x M) when ta; b is op(B) (K x N), stored transposed (N x K)
    when tb."""
    import torch

    from fp32_gemm_rm_amd.binding import sgemm_rm_op_strided_batched_ex

    dA = _stored_on_device(np.ascontiguousarray(a.T) if ta else a, lda)
    dB = _stored_on_device(np.ascontiguousarray(b.T) if tb else b, ldb)
    dC = torch.from_numpy(np.ascontiguousarray(c)).to("cuda")
    s = torch.cuda.current_stream()
    sgemm_rm_op_strided_batched_ex(ta, tb, M, N, K, alpha, dA.data_ptr(), lda, 0, dB.data_ptr(), ldb, 0, beta,
                                   dC.data_ptr(), N, 0, 1, s.cuda_stream, variant)
    s.synchronize()
    out = dC.cpu().numpy()
    del dA, dB, dC
    torch.cuda.empty_cache()
    return out


@pytest.mark.parametrize("tb", [0, 1])
@pytest.mark.parametrize("M,N,K", [(256, 512, 16 * 9), (512, 256, 48), (256, 256, 16 * 40), (256, 512, 16 * 9 + 5)])
def test_direct_and_staged_integer_exact(oracle, M, N, K, tb):
    print(f"[direct] {M}x{N}x{K} tb={tb} huge ld {HUGE_LD}", flush=True)
    a = integer_matrix(M, K, -4, 4, seed=M + K)
    b = integer_matrix(K, N, -4, 4, seed=N + K)
    c = integer_matrix(M, N, -4, 4, seed=M + N)
    ref, _ = oracle.full(M, N, K, -1.5, a.reshape(-1), K, b.reshape(-1), N, 0.5, c.reshape(-1), N, with_absab=False)
    # leading dimensions that are multiples of 4 (16-byte rows): the direct pipeline
    lda_small, ldb_small = _ld4(K) + 4, _ld4(K if tb else N) + 4
    direct = _run(M, N, K, a, lda_small, b, ldb_small, tb, c, -1.5, 0.5)
    # A's rows HUGE_LD apart: the register-staged pipeline (and B^T's too, when tb)
    staged = _run(M, N, K, a, HUGE_LD, b, HUGE_LD if tb else ldb_small, tb, c, -1.5, 0.5)
    for name, out in (("direct", direct), ("staged", staged)):
        got = c_window(out, M, N, N).astype(np.float64)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{name}: {len(bad)} mismatches, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("M,N,K", [(256, 256, 16 * 33), (512, 256, 16 * 20)])
def test_direct_and_staged_same_bits(M, N, K):
    """Random inputs: the two pipelines add the same products in the same order."""
    rng = np.random.default_rng(11)
    a = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    b = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    c = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    direct = _run(M, N, K, a, _ld4(K), b, N, 0, c, 1.25, -0.75)
    staged = _run(M, N, K, a, HUGE_LD, b, N, 0, c, 1.25, -0.75)
    assert np.array_equal(direct.view(np.uint32), staged.view(np.uint32))


# (M, N, K, ta, tb): remainders past the full 256 x 256 tiles of at least 16 run as guarded
# direct tiles, thinner ones as thin strips (rows 7 past 512; the last 2 columns of N = 274,
# which the guarded tiles along n leave to a strip since their limit is a multiple of 4)
GUARDED = [(256 + 40, 512 + 24, 144, 0, 0), (512 + 7, 256 + 100, 160, 0, 0), (256 + 16, 256 + 18, 48, 0, 0),
           (300, 520, 64, 1, 0), (300, 520, 64, 0, 1), (260 + 24, 256 + 36, 96, 1, 1)]


@pytest.mark.parametrize("M,N,K,ta,tb", GUARDED)
def test_direct_guarded_tiles_integer_exact(oracle, M, N, K, ta, tb):
    """Guarded direct tiles against the oracle, and against the register-staged path (rows of
    A HUGE_LD apart: scalar edge tiles or thin strips there), bit for bit; C's padding columns
    untouched is implied by comparing whole rows of width N."""
    print(f"[direct] guarded {M}x{N}x{K} ta={ta} tb={tb}", flush=True)
    a = integer_matrix(M, K, -4, 4, seed=M + 7 * K)
    b = integer_matrix(K, N, -4, 4, seed=N + 7 * K)
    c = integer_matrix(M, N, -4, 4, seed=M + 7 * N)
    ref, _ = oracle.full(M, N, K, 1.5, a.reshape(-1), K, b.reshape(-1), N, -0.5, c.reshape(-1), N, with_absab=False)
    lda = _ld4(M if ta else K) + 4
    ldb = _ld4(K if tb else N) + 4
    direct = _run(M, N, K, a, lda, b, ldb, tb, c, 1.5, -0.5, ta)
    got = c_window(direct, M, N, N).astype(np.float64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"direct: {len(bad)} mismatches, first at {bad[:3].tolist()}"
    if not ta:  # the register-staged 256 path, with A's rows too far apart for LDS-DMA
        staged = _run(M, N, K, a, HUGE_LD, b, ldb, tb, c, 1.5, -0.5, ta)
        got = c_window(staged, M, N, N).astype(np.float64)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"staged: {len(bad)} mismatches, first at {bad[:3].tolist()}"


# (M, N, K, ta, tb) on the 128 configuration, more than 256 tiles (its two-workgroup form):
# full tiles (272), guarded rows and columns with the last 2 columns of N = 2090 in a thin
# strip, A or B stored transposed, and a 12-row thin strip below the tiles
DIRECT128 = [(17 * 128, 16 * 128, 144, 0, 0), (2100, 2090, 160, 0, 0), (2100, 2088, 96, 1, 0),
             (2100, 2088, 96, 0, 1), (2060, 2100, 48, 1, 1)]


@pytest.mark.parametrize("M,N,K,ta,tb", DIRECT128)
def test_direct_128_integer_exact(oracle, M, N, K, ta, tb):
    """The 128 configuration's direct loop against the oracle, bit for bit."""
    print(f"[direct] 128 {M}x{N}x{K} ta={ta} tb={tb}", flush=True)
    a = integer_matrix(M, K, -4, 4, seed=M + 3 * K)
    b = integer_matrix(K, N, -4, 4, seed=N + 3 * K)
    c = integer_matrix(M, N, -4, 4, seed=M + 3 * N)
    ref, _ = oracle.full(M, N, K, -1.5, a.reshape(-1), K, b.reshape(-1), N, 0.5, c.reshape(-1), N, with_absab=False)
    lda = _ld4(M if ta else K) + 4
    ldb = _ld4(K if tb else N) + 4
    out = _run(M, N, K, a, lda, b, ldb, tb, c, -1.5, 0.5, ta, T128)
    got = c_window(out, M, N, N).astype(np.float64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("ta", [0, 1])
def test_direct_128_and_staged_same_bits(ta):
    """Random inputs on the 128 configuration's two-workgroup form: the direct loop (rows
    16-byte aligned) and the register-staged one (a leading dimension of A one float
    longer) add the same products in the same order, with A stored along k or along m."""
    M, N, K = 17 * 128, 16 * 128, 16 * 20
    rng = np.random.default_rng(12 + ta)
    a = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    b = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    c = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    ld = M if ta else K
    direct = _run(M, N, K, a, ld, b, N, 0, c, 1.25, -0.75, ta, T128)
    staged = _run(M, N, K, a, ld + 1, b, N, 0, c, 1.25, -0.75, ta, T128)
    assert np.array_equal(direct.view(np.uint32), staged.view(np.uint32))


# (M, N, K, ta, tb) on the 64 configuration, mostly more than 256 tiles: full tiles (272), thin
# strips on both sides (remainders 12 and 2), guarded rows and columns with B^T and with
# A^T, a single K-tile (fewer than the stages), and K a multiple of 16 but not of 32
DIRECT64 = [(17 * 64, 16 * 64, 96, 0, 0), (1100, 1090, 160, 0, 0), (1130, 1110, 64, 0, 1), (1060, 1060, 32, 0, 0),
            (1130, 1110, 64, 1, 0), (1100, 1100, 48, 0, 0),
            # one tile per CU: 256 full tiles, and 256 with guarded rows and columns
            (1024, 1024, 96, 0, 0), (1000, 1000, 64, 0, 0),
            # a partial last K-tile (through registers): one tile per CU, B^T, A^T B^T, and K
            # below one K-tile (no direct K-tile at all)
            (1024, 1024, 999, 0, 0), (1060, 1000, 40, 0, 1), (17 * 64, 16 * 64, 70, 1, 1), (1000, 1100, 21, 1, 0)]


@pytest.mark.parametrize("M,N,K,ta,tb", DIRECT64)
def test_direct_64_integer_exact(oracle, M, N, K, ta, tb):
    """The 64 configuration's two-workgroup form against the oracle, bit for bit."""
    print(f"[direct] 64 {M}x{N}x{K} ta={ta} tb={tb}", flush=True)
    a = integer_matrix(M, K, -4, 4, seed=M + 5 * K)
    b = integer_matrix(K, N, -4, 4, seed=N + 5 * K)
    c = integer_matrix(M, N, -4, 4, seed=M + 5 * N)
    ref, _ = oracle.full(M, N, K, 1.5, a.reshape(-1), K, b.reshape(-1), N, -0.5, c.reshape(-1), N, with_absab=False)
    lda = _ld4(M if ta else K) + 4
    ldb = _ld4(K if tb else N) + 4
    out = _run(M, N, K, a, lda, b, ldb, tb, c, 1.5, -0.5, ta, T64)
    got = c_window(out, M, N, N).astype(np.float64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"


def test_direct_64_and_staged_same_bits():
    """Random inputs on the 64 configuration's two-workgroup form: the direct loop and the
    register-staged one (lda = K + 1) add the same products in the same order, K-split
    partials included."""
    M, N, K = 17 * 64, 16 * 64, 32 * 9
    rng = np.random.default_rng(13)
    a = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    b = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    c = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    direct = _run(M, N, K, a, K, b, N, 0, c, 1.25, -0.75, 0, T64)
    staged = _run(M, N, K, a, K + 1, b, N, 0, c, 1.25, -0.75, 0, T64)
    assert np.array_equal(direct.view(np.uint32), staged.view(np.uint32))


# (variant, M, N, K, ta, tb): the 192 configuration (full tiles; guarded rows and columns;
# A^T or B^T; thin strips of 7 and 3) and the 128 one's one-layer form (one workgroup of
# 4 x 2 wavefronts per CU: full tiles, guarded A^T B^T, thin strips of 9 and 2)
DIRECT_MORE = [(T192, 3 * 192, 2 * 192, 144, 0, 0), (T192, 3 * 192 + 40, 2 * 192 + 20, 96, 0, 0),
               (T192, 420, 400, 64, 1, 0), (T192, 400, 420, 48, 0, 1), (T192, 2 * 192 + 7, 192 + 3, 64, 0, 0),
               (T128, 3 * 128, 2 * 128, 144, 0, 0), (T128, 300, 296, 64, 1, 1), (T128, 2 * 128 + 9, 3 * 128 + 2, 48, 0, 0)]


@pytest.mark.parametrize("variant,M,N,K,ta,tb", DIRECT_MORE)
def test_direct_192_and_128_one_layer_integer_exact(oracle, variant, M, N, K, ta, tb):
    """The 192 configuration's and the 128 one-layer form's direct loops against the oracle,
    bit for bit."""
    print(f"[direct] variant {variant} {M}x{N}x{K} ta={ta} tb={tb}", flush=True)
    a = integer_matrix(M, K, -4, 4, seed=M + 9 * K)
    b = integer_matrix(K, N, -4, 4, seed=N + 9 * K)
    c = integer_matrix(M, N, -4, 4, seed=M + 9 * N)
    ref, _ = oracle.full(M, N, K, -1.5, a.reshape(-1), K, b.reshape(-1), N, 0.5, c.reshape(-1), N, with_absab=False)
    lda = _ld4(M if ta else K) + 4
    ldb = _ld4(K if tb else N) + 4
    out = _run(M, N, K, a, lda, b, ldb, tb, c, -1.5, 0.5, ta, variant)
    got = c_window(out, M, N, N).astype(np.float64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("variant,M,N", [(T192, 2 * 192, 3 * 192), (T128, 2 * 128, 2 * 128)])
def test_direct_192_and_128_one_layer_same_bits(variant, M, N):
    """Random inputs: the direct loop and the register-staged one (lda = K + 1) give the same
    bits on the 192 configuration and the 128 one-layer form."""
    K = 16 * 21
    rng = np.random.default_rng(14)
    a = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    b = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    c = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    direct = _run(M, N, K, a, K, b, N, 0, c, 1.25, -0.75, 0, variant)
    staged = _run(M, N, K, a, K + 1, b, N, 0, c, 1.25, -0.75, 0, variant)
    assert np.array_equal(direct.view(np.uint32), staged.view(np.uint32))
