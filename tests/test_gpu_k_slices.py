"""K slices: products of few 64 x 64 tiles and long K, split along K over many workgroups.

With a workspace, a single product whose 64 x 64 tiles would leave most CUs idle has each
tile's K range cut into S contiguous slices, one workgroup each; the raw partial tiles go
to the workspace and a second kernel adds them in slice order and applies alpha and beta
(the deterministic split-K for small outputs).  The result must match the oracle like any
other path: bit for bit on integer inputs (every order of the sums is exact), within the
bound on random ones, the same on every run, with beta = 0 not reading C, and C's padding
untouched.  Shapes: one tile (S = 256), 16 tiles, guarded tiles on both sides, a K tail,
transposed operands, and the default path's choice against the forced 64 configuration.
"""
import numpy as np
import pytest

from fp32_gemm_rm_amd.workloads import C_PAD_SENTINEL, integer_matrix, make_inputs, pad_rows

from .parity import assert_within_bound, c_window, check_padding, device

pytestmark = pytest.mark.gpu

WS_BYTES = 128 << 20
# (M, N, K): every one takes K slices on the default path with a workspace
SHAPES = [(64, 64, 262144), (256, 256, 65536), (210, 148, 30000), (128, 192, 20001), (512, 512, 16384)]


@pytest.fixture(scope="module")
def ws():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp32_gemm_rm_amd import load_library

    load_library()
    return torch.empty(WS_BYTES, dtype=torch.uint8, device="cuda")


def _stored(x, trans, ld, pad):
    y = np.ascontiguousarray(x.T) if trans else x
    return pad_rows(y, ld, pad)


def _run(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, ta, tb, variant, ws):
    import torch

    from fp32_gemm_rm_amd import sgemm_rm_op_strided_batched_ws

    dA, dB, dC = device(A), device(B), device(C)
    s = torch.cuda.current_stream()
    sgemm_rm_op_strided_batched_ws(ta, tb, M, N, K, alpha, dA.data_ptr(), lda, 0, dB.data_ptr(), ldb, 0, beta,
                                   dC.data_ptr(), ldc, 0, 1, ws.data_ptr() if ws is not None else None,
                                   WS_BYTES if ws is not None else 0, s.cuda_stream, variant)
    s.synchronize()
    return dC.cpu().numpy()


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_workspace_size_asks_for_k_slices(ws, M, N, K):
    from fp32_gemm_rm_amd import sgemm_rm_workspace_size

    assert sgemm_rm_workspace_size(M, N, K, 1) == WS_BYTES
    assert sgemm_rm_workspace_size(M, N, K, 2) == 0  # batches never slice


@pytest.mark.parametrize("variant", [0, 7])  # default path, the 64 configuration forced
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_k_slices_integer_exact(oracle, ws, M, N, K, variant):
    print(f"[slices] {M}x{N}x{K} variant {variant}", flush=True)
    lda, ldb, ldc = K + 4, N + 4, N + 1
    a = integer_matrix(M, K, -4, 4, seed=M + 5 * K)
    b = integer_matrix(K, N, -4, 4, seed=N + 5 * K)
    c = integer_matrix(M, N, -4, 4, seed=M + 5 * N)
    A, B, C = pad_rows(a, lda, np.nan), pad_rows(b, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
    ref, _ = oracle.full(M, N, K, -1.5, A, lda, B, ldb, 0.5, C, ldc, with_absab=False)
    out = _run(M, N, K, -1.5, A, lda, B, ldb, 0.5, C, ldc, 0, 0, variant, ws)
    got = c_window(out, M, N, ldc).astype(np.float64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"
    check_padding(out, C, M, N, ldc)
    again = _run(M, N, K, -1.5, A, lda, B, ldb, 0.5, C, ldc, 0, 0, variant, ws)
    assert np.array_equal(out.view(np.uint32), again.view(np.uint32)), "not deterministic"


@pytest.mark.parametrize("M,N,K", SHAPES[:4])
def test_k_slices_random_bound_beta_zero(oracle, ws, M, N, K):
    """Random inputs within the bound; beta = 0 over a NaN C (C is not read)."""
    lda, ldb, ldc = K, N, N
    A, B, C = make_inputs(M, N, K, lda, ldb, ldc, "uniform", seed=M + N, c_init="nan")
    ref, S = oracle.full(M, N, K, 1.25, A, lda, B, ldb, 0.0, C, ldc)
    out = _run(M, N, K, 1.25, A, lda, B, ldb, 0.0, C, ldc, 0, 0, 0, ws)
    assert_within_bound(c_window(out, M, N, ldc), ref, S, f"{M}x{N}x{K}")


@pytest.mark.parametrize("ta,tb", [(0, 1), (1, 0), (1, 1)])
def test_k_slices_transposed_integer_exact(oracle, ws, ta, tb):
    M, N, K = 210, 148, 30000
    lda, ldb, ldc = (M if ta else K) + 4, (K if tb else N) + 4, N + 1
    a = integer_matrix(M, K, -4, 4, seed=7 + ta)
    b = integer_matrix(K, N, -4, 4, seed=9 + tb)
    c = integer_matrix(M, N, -4, 4, seed=11)
    A, B, C = _stored(a, ta, lda, np.nan), _stored(b, tb, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
    ref, _ = oracle.full(M, N, K, 2.0, a.reshape(-1), K, b.reshape(-1), N, -1.0, C, ldc, with_absab=False)
    out = _run(M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, ta, tb, 0, ws)
    got = c_window(out, M, N, ldc).astype(np.float64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"op {ta}{tb}: {len(bad)} mismatches, first at {bad[:3].tolist()}"
    check_padding(out, C, M, N, ldc)
