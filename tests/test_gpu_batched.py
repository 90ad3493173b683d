"""GPU parity of the strided-batched entry points against the CPU oracle, entry by entry.

The batched form follows "GPU-accelerated matrix computation ..." section 4.2
(strided batch, strides M*K, K*N, M*N, batchCount 1024 of 64 x 64 products);
every entry must match the oracle's result for that entry alone, within the
same bound as a single GEMM, and nothing outside the entries' C windows may be
written.
"""
import numpy as np
import pytest

from fp32_gemm_rm_amd.workloads import BATCHED_BY_NAME, C_PAD_SENTINEL, make_batched_inputs

from .parity import assert_within_bound, device

pytestmark = pytest.mark.gpu

VARIANTS = {"naive": 1, "lds_tiled": 2, "regblock": 3, "mfma": 4, "auto": 0}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run_batched(M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC, batch, variant):
    import torch

    from fp32_gemm_rm_amd import sgemm_rm_strided_batched_ex

    dA, dB, dC = device(A), device(B), device(C)
    s = torch.cuda.current_stream()
    sgemm_rm_strided_batched_ex(M, N, K, alpha, dA.data_ptr(), lda, sA, dB.data_ptr(), ldb, sB, beta,
                                dC.data_ptr(), ldc, sC, batch, s.cuda_stream, variant)
    s.synchronize()
    return dC.cpu().numpy()


def _entry(buf, off, rows, cols, ld):
    return np.stack([buf[off + i * ld: off + i * ld + cols] for i in range(rows)]) if rows else np.zeros((0, cols))


def _check_entries(oracle, out, M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC, entries):
    nA, nB, nC = (M - 1) * lda + K, (K - 1) * ldb + N, (M - 1) * ldc + N
    for b in entries:
        ref, S = oracle.full(M, N, K, alpha, A[b * sA: b * sA + nA], lda, B[b * sB: b * sB + nB], ldb, beta,
                             C[b * sC: b * sC + nC], ldc)
        assert_within_bound(_entry(out, b * sC, M, N, ldc), ref, S, f"entry {b}")
    # nothing outside the C windows changed
    mask = np.ones(out.size, bool)
    for b in entries:
        for i in range(M):
            mask[b * sC + i * ldc: b * sC + i * ldc + N] = False
    assert np.array_equal(out[mask].view(np.uint32), C[mask].view(np.uint32))


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize(
    "M,N,K,batch,share_b",
    [(64, 64, 64, 37, False), (70, 33, 129, 5, False), (130, 257, 17, 3, True), (5, 300, 64, 9, False),
     # 9 guarded 128^2 tiles x 30 entries = 270 > 256: the 128 configuration's two-workgroup form
     (300, 300, 33, 30, False)],
)
def test_batched_parity(oracle, variant, M, N, K, batch, share_b):
    lda, ldb, ldc = K + 3, N + 1, N + 2
    sA = M * lda + 7  # gaps between entries (NaN in A and B, the sentinel in C)
    sB = 0 if share_b else K * ldb + 5
    sC = M * ldc + 11
    A, B, C = make_batched_inputs(batch, M, N, K, lda, ldb, ldc, sA, sB, sC, "uniform", seed=M + N + batch,
                                  c_init="random")
    out = _run_batched(M, N, K, 1.5, A, lda, sA, B, ldb, sB, -0.5, C, ldc, sC, batch, VARIANTS[variant])
    _check_entries(oracle, out, M, N, K, 1.5, A, lda, sA, B, ldb, sB, -0.5, C, ldc, sC, range(batch))


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_batched_aligned_rows_odd_strides(oracle, variant):
    """Leading dimensions that are multiples of 4 on 16-byte aligned buffers, with batch
    strides that are not: entry 0 would allow 128-bit loads, entries 1.. do not, so every
    launcher must take the scalar loads for the whole batch."""
    M, N, K, batch = 70, 96, 132, 4
    lda, ldb, ldc = K, N, N
    sA, sB, sC = M * lda + 1, K * ldb + 3, M * ldc + 5
    A, B, C = make_batched_inputs(batch, M, N, K, lda, ldb, ldc, sA, sB, sC, "uniform", seed=77, c_init="random")
    out = _run_batched(M, N, K, 1.5, A, lda, sA, B, ldb, sB, -0.5, C, ldc, sC, batch, VARIANTS[variant])
    _check_entries(oracle, out, M, N, K, 1.5, A, lda, sA, B, ldb, sB, -0.5, C, ldc, sC, range(batch))


@pytest.mark.parametrize("variant", [7, 0])  # the 64 x 64 configuration forced, and the default path
def test_batched_fused_right_strip(oracle, variant):
    """Entries whose right strip runs inside the 64 x 64 tiles (16 tile columns, 5 strip
    columns, K >= 640, guarded tile rows): each entry's strip reads its own B columns."""
    M, N, K, batch = 130, 16 * 64 + 5, 700, 3
    lda, ldb, ldc = K + 3, N + 1, N + 2
    sA, sB, sC = M * lda + 7, K * ldb + 5, M * ldc + 11
    A, B, C = make_batched_inputs(batch, M, N, K, lda, ldb, ldc, sA, sB, sC, "uniform", seed=31, c_init="random")
    out = _run_batched(M, N, K, 1.5, A, lda, sA, B, ldb, sB, -0.5, C, ldc, sC, batch, variant)
    _check_entries(oracle, out, M, N, K, 1.5, A, lda, sA, B, ldb, sB, -0.5, C, ldc, sC, range(batch))


def test_batched_more_entries_than_one_launch(oracle):
    """70000 entries: two launches (65535 + 4465); integer inputs, checked bit for bit at the seams."""
    import torch

    M = N = K = 4
    batch = 70000
    gen = torch.Generator().manual_seed(9)
    A = torch.randint(-3, 4, (batch * 16,), generator=gen).float().numpy()
    B = torch.randint(-3, 4, (batch * 16,), generator=gen).float().numpy()
    C = torch.randint(-3, 4, (batch * 16,), generator=gen).float().numpy()
    out = _run_batched(M, N, K, 2.0, A, 4, 16, B, 4, 16, -1.0, C, 4, 16, batch, 0)
    for b in (0, 1, 65534, 65535, 65536, batch - 1):
        ref, _ = oracle.full(M, N, K, 2.0, A[b * 16:(b + 1) * 16], 4, B[b * 16:(b + 1) * 16], 4, -1.0,
                             C[b * 16:(b + 1) * 16], 4)
        np.testing.assert_array_equal(out[b * 16:(b + 1) * 16].reshape(4, 4).astype(np.float64), ref)


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_batched_workload(oracle, variant):
    """The 1024 x (64 x 64 x 64) batch, every entry against the oracle."""
    w = BATCHED_BY_NAME["sgemm_batched_1024x64"]
    M, N, K = w.M, w.N, w.K
    A, B, C = make_batched_inputs(w.batch, M, N, K, K, N, N, M * K, K * N, M * N, w.dist, w.seed, "zeros")
    out = _run_batched(M, N, K, w.alpha, A, K, M * K, B, N, K * N, w.beta, C, N, M * N, w.batch, VARIANTS[variant])
    _check_entries(oracle, out, M, N, K, w.alpha, A, K, M * K, B, N, K * N, w.beta, C, N, M * N, range(w.batch))


def test_batched_alpha_zero_scales_every_entry():
    M, N, K, batch = 17, 9, 5, 6
    lda, ldb, ldc = K, N, N + 1
    sC = M * ldc + 3
    _, _, C = make_batched_inputs(batch, M, N, K, lda, ldb, ldc, 0, 0, sC, "uniform", seed=4, c_init="random")
    A = np.full(M * lda, np.nan, np.float32)
    B = np.full(K * ldb, np.nan, np.float32)
    out = _run_batched(M, N, K, 0.0, A, lda, 0, B, ldb, 0, -0.5, C, ldc, sC, batch, 0)
    for b in range(batch):
        want = (np.float32(-0.5) * _entry(C, b * sC, M, N, ldc)).astype(np.float32)
        np.testing.assert_array_equal(_entry(out, b * sC, M, N, ldc), want)


def test_batched_tensor_binding():
    import torch

    from fp32_gemm_rm_amd import sgemm_batched

    g = torch.Generator(device="cuda").manual_seed(3)
    A = torch.randint(-3, 4, (7, 50, 40), generator=g, device="cuda").float()
    B = torch.randint(-3, 4, (7, 40, 30), generator=g, device="cuda").float()
    C = torch.full((7, 50, 30), float("nan"), device="cuda")
    sgemm_batched(A, B, C, 1.0, 0.0)
    torch.cuda.synchronize()
    want = torch.bmm(A.double().cpu(), B.double().cpu()).float()
    assert torch.equal(C.cpu(), want)


@pytest.mark.parametrize("tiles,M,N,K,batch", [(256, 256 + 40, 512 + 24, 144, 3), (256, 300, 256 + 7, 64, 3),
                                                 (128, 300, 296, 64, 40), (128, 2 * 128 + 9, 3 * 128, 48, 50),
                                                 (64, 150, 140, 64, 50), (64, 150, 140, 68, 50), (64, 300, 200, 96, 2),
                                                 (192, 2 * 192 + 40, 192 + 20, 48, 4), (128, 300, 296, 64, 3)])
def test_batched_direct_guarded_tiles(oracle, tiles, M, N, K, batch):
    """The 256 x 256 configuration, the 192 one, and the 128 and 64 ones with more than 256
    tiles over the batch (their two-workgroup forms) or fewer, forced on entries with 16-byte aligned rows and strides: the
    LDS-DMA K loop with guarded tiles (256: remainders of 40 rows and 24 columns; 44 rows;
    128: 44 rows and 40 columns; 64: 22 rows, also with a partial last K-tile, and 44 rows
    at one tile per CU) and thin strips (7 columns; 9 rows; 12 columns; 8 columns), each
    entry reading its own operands between NaN gaps."""
    from fp32_gemm_rm_amd import TILE_VARIANTS

    lda, ldb, ldc = K + 4, (N + 7) // 4 * 4, N + 2
    sA, sB, sC = M * lda + 8, K * ldb + 4, M * ldc + 11
    A, B, C = make_batched_inputs(batch, M, N, K, lda, ldb, ldc, sA, sB, sC, "uniform", seed=M + K,
                                  c_init="random")
    out = _run_batched(M, N, K, 1.5, A, lda, sA, B, ldb, sB, -0.5, C, ldc, sC, batch, TILE_VARIANTS[tiles])
    _check_entries(oracle, out, M, N, K, 1.5, A, lda, sA, B, ldb, sB, -0.5, C, ldc, sC, range(batch))
