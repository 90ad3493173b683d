"""GPU parity of the transposed-operand and column-major forms, through the C ABI.

C = alpha * op(A) * op(B) + beta * C with op = N or T on either operand, row-major
(sgemm_rm_op and its batched form) and column-major (sgemm_cm and its batched form).
Each case draws the logical op(A) (M x K) and op(B) (K x N), lays them out in the
storage the call describes (transposed and/or column-major, padded leading
dimensions with NaN in the padding), and compares the result with the oracle run
on the logical row-major matrices: bit for bit on integer inputs, within the bound
on random ones.  Storage layout is data movement only; the oracle computes the
plain row-major product.
"""
import numpy as np
import pytest

from fp32_gemm_rm_amd.workloads import C_PAD_SENTINEL, integer_matrix, make_inputs, pad_rows

from .parity import assert_within_bound, device, edge_shapes

pytestmark = pytest.mark.gpu

VARIANTS = {"naive": 1, "lds_tiled": 2, "regblock": 3, "mfma": 4, "auto": 0}
ORIENTATIONS = {"nn": (0, 0), "nt": (0, 1), "tn": (1, 0), "tt": (1, 1)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp32_gemm_rm_amd import load_library

    load_library()


def store(mat, trans, cm, ld, fill):
    """Flat buffer holding the logical matrix ``mat`` as the call reads it: transposed
    when ``trans``, and column-major (the row-major layout of the transpose) when ``cm``."""
    stored = mat.T if trans else mat
    return pad_rows(np.ascontiguousarray(stored.T if cm else stored), ld, fill)


def min_ld(rows, cols, trans, cm):
    """Smallest leading dimension of a logical rows x cols operand in the given storage."""
    s_rows, s_cols = (cols, rows) if trans else (rows, cols)
    return max(1, s_rows if cm else s_cols)


def read_c(buf, M, N, ldc, cm):
    """Logical M x N window of an output buffer."""
    if cm:
        return buf.reshape(-1)[: N * ldc].reshape(N, ldc)[:, :M].T
    return buf.reshape(-1)[: M * ldc].reshape(M, ldc)[:, :N]


def c_padding_unchanged(out, C, M, N, ldc, cm):
    rows, cols = (N, M) if cm else (M, N)
    if ldc > cols and rows > 0:
        a = out.reshape(-1)[: rows * ldc].reshape(rows, ldc)[:, cols:].view(np.uint32)
        b = C.reshape(-1)[: rows * ldc].reshape(rows, ldc)[:, cols:].view(np.uint32)
        return np.array_equal(a, b)
    return True


def run_op(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant, cm=False, batch=1, strides=(0, 0, 0)):
    """One call of the general row-major or column-major entry point on device copies."""
    import torch

    from fp32_gemm_rm_amd import sgemm_cm_strided_batched_ex, sgemm_rm_op_strided_batched_ex

    dA, dB, dC = device(A), device(B), device(C)
    fn = sgemm_cm_strided_batched_ex if cm else sgemm_rm_op_strided_batched_ex
    s = torch.cuda.current_stream()
    fn(ta, tb, M, N, K, alpha, dA.data_ptr(), lda, strides[0], dB.data_ptr(), ldb, strides[1], beta,
       dC.data_ptr(), ldc, strides[2], batch, s.cuda_stream, variant)
    s.synchronize()
    return dC.cpu().numpy()


def oracle_logical(oracle, M, N, K, alpha, a, b, beta, c):
    """Oracle on the logical row-major matrices (dense, no padding)."""
    return oracle.full(M, N, K, alpha, a.reshape(-1), max(K, 1), b.reshape(-1), max(N, 1), beta,
                       c.reshape(-1), max(N, 1))


@pytest.mark.parametrize("cm", [False, True], ids=["rm", "cm"])
@pytest.mark.parametrize("orient", list(ORIENTATIONS))
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_edge_shapes_integer_exact(oracle, variant, orient, cm):
    """Ragged shapes around the tile sizes, integer inputs, every orientation and storage
    order: bit-exact, padding of C untouched."""
    ta, tb = ORIENTATIONS[orient]
    print(f"[transposed] edge shapes {variant} {orient} {'cm' if cm else 'rm'}", flush=True)
    for t, (M, N, K) in enumerate(edge_shapes()[::2]):
        a = integer_matrix(M, K, -4, 4, seed=900 + t)
        b = integer_matrix(K, N, -4, 4, seed=1000 + t)
        c = integer_matrix(M, N, -4, 4, seed=1100 + t)
        lda = min_ld(M, K, ta, cm) + (t % 5)
        ldb = min_ld(K, N, tb, cm) + (t % 3)
        ldc = min_ld(M, N, False, cm) + 1 + (t % 4)
        A, B = store(a, ta, cm, lda, np.nan), store(b, tb, cm, ldb, np.nan)
        C = store(c, False, cm, ldc, C_PAD_SENTINEL)
        out = run_op(ta, tb, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, VARIANTS[variant], cm=cm)
        ref, _ = oracle_logical(oracle, M, N, K, 2.0, a, b, -1.0, c)
        got = read_c(out, M, N, ldc, cm).astype(np.float64)
        assert np.array_equal(got, ref), f"shape {(M, N, K)} lds {(lda, ldb, ldc)}"
        assert c_padding_unchanged(out, C, M, N, ldc, cm), f"C padding written, shape {(M, N, K)}"


@pytest.mark.parametrize("variant", [7, 0])  # the 64 configuration forced, the default path
def test_column_major_fused_right_strip(oracle, variant):
    """A column-major NN call runs as the row-major product C^T = B^T A^T, whose right strip
    (columns past 16 tile columns of 64) is computed inside the 64 x 64 tiles at K >= 640:
    here the strip is the last 5 rows of the column-major C."""
    M, N, K = 16 * 64 + 5, 200, 700
    a = integer_matrix(M, K, -4, 4, seed=71)
    b = integer_matrix(K, N, -4, 4, seed=72)
    c = integer_matrix(M, N, -4, 4, seed=73)
    lda, ldb, ldc = M + 3, K + 1, M + 2
    A, B, C = store(a, False, True, lda, np.nan), store(b, False, True, ldb, np.nan), store(c, False, True, ldc,
                                                                                             C_PAD_SENTINEL)
    out = run_op(0, 0, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, variant, cm=True)
    ref, _ = oracle_logical(oracle, M, N, K, 2.0, a, b, -1.0, c)
    got = read_c(out, M, N, ldc, True).astype(np.float64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"
    assert c_padding_unchanged(out, C, M, N, ldc, True)


@pytest.mark.parametrize("orient", ["nt", "tn", "tt"])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_ragged_random_bound(oracle, variant, orient):
    """The ragged 1000 x 1030 x 999 problem (alpha 1.5, beta -0.5, padded leading
    dimensions) with transposed operands, within the bound."""
    ta, tb = ORIENTATIONS[orient]
    M, N, K = 1000, 1030, 999
    a_, b_, c_ = make_inputs(M, N, K, K, N, N, "normal", seed=31, c_init="random")
    a, b, c = a_.reshape(M, K), b_.reshape(K, N), c_.reshape(M, N)
    lda, ldb, ldc = min_ld(M, K, ta, False) + 8, min_ld(K, N, tb, False) + 10, N + 10
    A, B, C = store(a, ta, False, lda, np.nan), store(b, tb, False, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
    out = run_op(ta, tb, M, N, K, 1.5, A, lda, B, ldb, -0.5, C, ldc, VARIANTS[variant])
    ref, S = oracle_logical(oracle, M, N, K, 1.5, a, b, -0.5, c)
    r = assert_within_bound(read_c(out, M, N, ldc, False), ref, S, f"{orient}/{variant}")
    assert c_padding_unchanged(out, C, M, N, ldc, False)
    print(f"[transposed] ragged {orient} {variant} max err/bound {r:.3g}", flush=True)


# Small shapes per forced MFMA tile configuration: several full tiles plus partial ones,
# guarded or thin (strips thinner than 16, or 4 for 32, and the last 1-3 rows or columns
# of a guarded remainder that is not a multiple of 4), and full tiles only (96 x 64; for
# 128, one layer of exact tiles (4 x 2 wavefronts), and 272 exact or 289 guarded ones (the
# two-workgroup form)).
TILE_SHAPES = [(256, 600, 520, 77), (256, 300, 270, 160), (256, 516, 259, 77), (192, 400, 390, 77), (192, 3 * 192 + 7, 232, 300),
               (128, 300, 290, 77), (128, 140, 290, 257), (128, 256, 384, 77), (128, 2176, 2048, 45),
               (128, 2100, 2090, 45),
               (128, 143, 265, 77), (64, 200, 150, 77), (64, 130, 70, 450), (64, 199, 141, 450), (64, 67, 73, 2100),
               (32, 100, 70, 77), (32, 103, 70, 77), (32, 96, 64, 77), (32, 40, 70, 449),
               (16, 100, 70, 77), (16, 33, 17, 1045)]


@pytest.mark.parametrize("orient", ["nt", "tn", "tt"])
@pytest.mark.parametrize("tiles,M,N,K", TILE_SHAPES)
def test_tile_configs_integer_exact(oracle, tiles, M, N, K, orient):
    """Every MFMA tile configuration with transposed operands: bit-exact on integer inputs."""
    from fp32_gemm_rm_amd import TILE_VARIANTS

    ta, tb = ORIENTATIONS[orient]
    a = integer_matrix(M, K, -4, 4, seed=M + K)
    b = integer_matrix(K, N, -4, 4, seed=N + K)
    c = integer_matrix(M, N, -4, 4, seed=M + N)
    lda, ldb, ldc = min_ld(M, K, ta, False) + 4, min_ld(K, N, tb, False) + 8, N + 3
    A, B, C = store(a, ta, False, lda, np.nan), store(b, tb, False, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
    out = run_op(ta, tb, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, TILE_VARIANTS[tiles])
    ref, _ = oracle_logical(oracle, M, N, K, 2.0, a, b, -1.0, c)
    got = read_c(out, M, N, ldc, False).astype(np.float64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"
    assert c_padding_unchanged(out, C, M, N, ldc, False)


@pytest.mark.parametrize("orient", ["nt", "tn", "tt"])
@pytest.mark.parametrize(
    "M,N,K",
    [
        (2048, 2048, 300),   # 128 x 128 tiles
        (4196, 4132, 77),    # 64 x 64 tiles plus edge strips, ragged K
        (4096, 4096, 17),    # 256 x 256 tiles, K just past one K-tile
        (1000, 1030, 99),    # 64 x 64 tiles, guarded partial rows, thin column strip
    ],
)
def test_default_path_integer_exact(oracle, M, N, K, orient):
    """The default path with transposed operands at shapes that select each tile
    configuration: bit-exact on integer inputs."""
    ta, tb = ORIENTATIONS[orient]
    a = integer_matrix(M, K, -4, 4, seed=M + K)
    b = integer_matrix(K, N, -4, 4, seed=N + K)
    c = integer_matrix(M, N, -4, 4, seed=M + N)
    lda, ldb, ldc = min_ld(M, K, ta, False) + 4, min_ld(K, N, tb, False) + 8, N + 3
    A, B, C = store(a, ta, False, lda, np.nan), store(b, tb, False, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
    out = run_op(ta, tb, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, VARIANTS["auto"])
    ref, _ = oracle_logical(oracle, M, N, K, 2.0, a, b, -1.0, c)
    got = read_c(out, M, N, ldc, False).astype(np.float64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"
    assert c_padding_unchanged(out, C, M, N, ldc, False)


@pytest.mark.parametrize("orient", ["nt", "tn", "tt"])
def test_headline_shape_full(oracle, orient):
    """4096^3 with transposed operands on the default path, normal inputs, beta = 1:
    every output within the bound."""
    import torch

    from fp32_gemm_rm_amd import sgemm

    ta, tb = ORIENTATIONS[orient]
    M = N = K = 4096
    print(f"[transposed] 4096^3 {orient}", flush=True)
    a_, b_, c_ = make_inputs(M, N, K, K, N, N, "normal", seed=4096 + ta + 2 * tb, c_init="random")
    a, b, c = a_.reshape(M, K), b_.reshape(K, N), c_.reshape(M, N)
    # transposed operands as transposed views of row-major device tensors
    dA = device(a.T).t() if ta else device(a)
    dB = device(b.T).t() if tb else device(b)
    dC = device(c)
    sgemm(dA, dB, dC, alpha=1.0, beta=1.0)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    ref, S = oracle.full(M, N, K, 1.0, a_, K, b_, N, 1.0, c_, N)
    r = assert_within_bound(out, ref, S, orient)
    print(f"[transposed] 4096^3 {orient}: every output, max err/bound {r:.3g}", flush=True)


@pytest.mark.parametrize("cm", [False, True], ids=["rm", "cm"])
@pytest.mark.parametrize("orient", list(ORIENTATIONS))
@pytest.mark.parametrize("variant", ["mfma", "regblock", "naive"])
def test_batched_integer_exact(oracle, variant, orient, cm):
    """Strided batches of transposed / column-major problems, with gaps between the
    entries (left untouched) and a shared B (stride 0) in the column-major case."""
    ta, tb = ORIENTATIONS[orient]
    M, N, K, batch = 130, 200, 77, 3
    lda, ldb, ldc = min_ld(M, K, ta, cm) + 3, min_ld(K, N, tb, cm) + 1, min_ld(M, N, False, cm) + 2
    a = [integer_matrix(M, K, -4, 4, seed=1200 + i) for i in range(batch)]
    b = [integer_matrix(K, N, -4, 4, seed=1300 + (0 if cm else i)) for i in range(batch)]
    c = [integer_matrix(M, N, -4, 4, seed=1400 + i) for i in range(batch)]
    As = [store(x, ta, cm, lda, np.nan) for x in a]
    Bs = [store(x, tb, cm, ldb, np.nan) for x in b]
    Cs = [store(x, False, cm, ldc, C_PAD_SENTINEL) for x in c]
    sA, sB, sC = len(As[0]) + 5, 0 if cm else len(Bs[0]) + 7, len(Cs[0]) + 11
    A = np.full(sA * batch, np.nan, np.float32)
    B = np.full(max(sB * batch, len(Bs[0])), np.nan, np.float32)
    C = np.full(sC * batch, C_PAD_SENTINEL, np.float32)
    for i in range(batch):
        A[i * sA: i * sA + len(As[i])] = As[i]
        B[i * sB: i * sB + len(Bs[i])] = Bs[i]
        C[i * sC: i * sC + len(Cs[i])] = Cs[i]
    out = run_op(ta, tb, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, VARIANTS[variant], cm=cm, batch=batch,
                 strides=(sA, sB, sC))
    for i in range(batch):
        ref, _ = oracle_logical(oracle, M, N, K, 2.0, a[i], b[i], -1.0, c[i])
        entry = out[i * sC: i * sC + len(Cs[i])]
        assert np.array_equal(read_c(entry, M, N, ldc, cm).astype(np.float64), ref), f"entry {i}"
        assert c_padding_unchanged(entry, Cs[i], M, N, ldc, cm), f"entry {i} padding"
        gap = out[i * sC + len(Cs[i]): (i + 1) * sC]
        assert np.all(gap == np.float32(C_PAD_SENTINEL)), f"gap after entry {i} written"


def test_cm_is_rm_of_transposes(oracle):
    """The column-major call on buffers X equals the row-major call on the same buffers
    with operands and M, N swapped (C^T = op(B)^T op(A)^T): bitwise, on random inputs."""
    import torch

    from fp32_gemm_rm_amd import sgemm_cm, sgemm_rm_op

    M, N, K = 300, 257, 129
    rng = np.random.default_rng(5)
    for ta, tb in ORIENTATIONS.values():
        lda, ldb, ldc = (K if ta else M) + 2, (N if tb else K) + 1, M + 3
        A = device(rng.standard_normal(lda * (M if ta else K)).astype(np.float32))
        B = device(rng.standard_normal(ldb * (K if tb else N)).astype(np.float32))
        C0 = rng.standard_normal(ldc * N).astype(np.float32)
        C1, C2 = device(C0), device(C0)
        s = torch.cuda.current_stream().cuda_stream
        sgemm_cm(ta, tb, M, N, K, 0.75, A.data_ptr(), lda, B.data_ptr(), ldb, 0.5, C1.data_ptr(), ldc, s)
        sgemm_rm_op(tb, ta, N, M, K, 0.75, B.data_ptr(), ldb, A.data_ptr(), lda, 0.5, C2.data_ptr(), ldc, s)
        torch.cuda.synchronize()
        assert torch.equal(C1, C2), (ta, tb)


def test_tensor_views(oracle):
    """The tensor-level call takes transposed views without copies: A.t() and B.t()
    of row-major tensors give the same result as the row-major call on copies."""
    import torch

    from fp32_gemm_rm_amd import sgemm

    M, N, K = 515, 333, 260
    a_, b_, _ = make_inputs(M, N, K, K, N, N, "uniform", seed=12)
    a, b = a_.reshape(M, K), b_.reshape(K, N)
    ref, S = oracle_logical(oracle, M, N, K, 1.0, a, b, 0.0, np.zeros((M, N), np.float32))
    for ta, tb in ORIENTATIONS.values():
        dA = device(a.T).t() if ta else device(a)
        dB = device(b.T).t() if tb else device(b)
        assert dA.stride(0 if ta else 1) == 1 and dB.stride(0 if tb else 1) == 1
        dC = torch.full((M, N), float("nan"), device="cuda")
        sgemm(dA, dB, dC)
        torch.cuda.synchronize()
        assert_within_bound(dC.cpu().numpy(), ref, S, f"views {(ta, tb)}")
