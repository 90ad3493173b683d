"""GPU parity of the stream-K path (the _ws calls with a workspace), through the C ABI.

SGEMM_RM_VARIANT_MFMA_T256 with a workspace runs stream-K wherever the 256 x 256 tiles
leave a partial wave of 256 workgroups, so small shapes exercise every part of it:
ranges shorter than one K-tile, ranges inside one tile, ranges over several tiles, tiles
written whole by one range, one-tile-per-workgroup tiles before the stream-K waves, and
the scalar edge tiles around them.  Integer inputs make every summation order exact, so
the comparison with the oracle is bit for bit; random inputs at 4608^3 (the default
path's own choice of stream-K) are checked at every output within the bound.
"""
import numpy as np
import pytest

from fp32_gemm_rm_amd.workloads import C_PAD_SENTINEL, integer_matrix, make_inputs, pad_rows

from .parity import assert_within_bound, c_window, check_padding, device

pytestmark = pytest.mark.gpu

T256 = 5
WS_BYTES = 2 * 256 * 256 * 256 * 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp32_gemm_rm_amd import load_library

    load_library()


@pytest.fixture(scope="module")
def workspace():
    import torch

    return torch.empty(WS_BYTES, dtype=torch.uint8, device="cuda")


def run_ws(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant, ws, ta=0, tb=0):
    import torch

    from fp32_gemm_rm_amd import sgemm_rm_op_strided_batched_ws

    dA, dB, dC = device(A), device(B), device(C)
    s = torch.cuda.current_stream()
    sgemm_rm_op_strided_batched_ws(ta, tb, M, N, K, alpha, dA.data_ptr(), lda, 0, dB.data_ptr(), ldb, 0, beta,
                                   dC.data_ptr(), ldc, 0, 1, ws.data_ptr() if ws is not None else None,
                                   ws.numel() if ws is not None else 0, s.cuda_stream, variant)
    s.synchronize()
    return dC.cpu().numpy()


@pytest.mark.parametrize(
    "M,N,K",
    [
        (512, 768, 300),      # 6 tiles: 256 ranges of under one K-tile, most of them empty
        (512, 768, 4000),     # 6 tiles, long K: each tile split over ~43 ranges
        (1024, 1280, 77),     # 20 tiles, ragged K
        (4352, 4352, 77),     # 289 tiles: 256 one-tile workgroups, 33 stream-K tiles (the partial wave)
        (4352 + 37, 4352 + 19, 40),  # the same with scalar edge tiles around them
        (4096, 4608, 200),    # 288 tiles: 32 in the partial wave, which alone is stream-K
        (1792, 10496, 200),   # 287 tiles: 31 in the partial wave, stream-K with the wave before it
        (6144, 5632, 40),     # 528 tiles: 256 one-tile workgroups, then 272 stream-K tiles (16 + 256)
    ],
)
def test_stream_k_integer_exact(oracle, workspace, M, N, K):
    lda, ldb, ldc = K + 4, N + 8, N + 3
    a = integer_matrix(M, K, -4, 4, seed=M + 2 * K)
    b = integer_matrix(K, N, -4, 4, seed=N + 3 * K)
    c = integer_matrix(M, N, -4, 4, seed=M + N + K)
    A, B, C = pad_rows(a, lda, np.nan), pad_rows(b, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
    print(f"[stream-k] {M}x{N}x{K}", flush=True)
    out = run_ws(M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, T256, workspace)
    ref, _ = oracle.full(M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc)
    got = c_window(out, M, N, ldc).astype(np.float64)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"
    check_padding(out, C, M, N, ldc)


@pytest.mark.parametrize("ta,tb", [(0, 1), (1, 0), (1, 1)])
def test_stream_k_transposed_integer_exact(oracle, workspace, ta, tb):
    M, N, K = 1024, 1280, 333
    a = integer_matrix(M, K, -4, 4, seed=7)
    b = integer_matrix(K, N, -4, 4, seed=8)
    c = integer_matrix(M, N, -4, 4, seed=9)
    A = np.ascontiguousarray(a.T if ta else a).reshape(-1)
    B = np.ascontiguousarray(b.T if tb else b).reshape(-1)
    lda, ldb = (M if ta else K), (K if tb else N)
    out = run_ws(M, N, K, 1.0, A, lda, B, ldb, 1.0, c.reshape(-1), N, T256, workspace, ta, tb)
    ref, _ = oracle.full(M, N, K, 1.0, a.reshape(-1), K, b.reshape(-1), N, 1.0, c.reshape(-1), N)
    np.testing.assert_array_equal(out.reshape(M, N).astype(np.float64), ref)


def test_stream_k_beta_zero_ignores_nan_c(oracle, workspace):
    M, N, K = 1024, 768, 200
    A, B, _ = make_inputs(M, N, K, K, N, N, "uniform", seed=21)
    C = np.full(M * N, np.nan, np.float32)
    out = run_ws(M, N, K, 1.5, A, K, B, N, 0.0, C, N, T256, workspace)
    ref, S = oracle.full(M, N, K, 1.5, A, K, B, N, 0.0, None, N)
    assert_within_bound(out.reshape(M, N), ref, S, "beta 0")


def test_stream_k_deterministic(workspace):
    """Two calls give the same bits; without a workspace the forced variant is the
    one-tile-per-workgroup path (also deterministic, other summation order)."""
    M, N, K = 1280, 1536, 1000
    A, B, C = make_inputs(M, N, K, K, N, N, "normal", seed=5, c_init="random")
    r1 = run_ws(M, N, K, 1.0, A, K, B, N, 0.5, C, N, T256, workspace)
    r2 = run_ws(M, N, K, 1.0, A, K, B, N, 0.5, C, N, T256, workspace)
    assert np.array_equal(r1.view(np.uint32), r2.view(np.uint32))
    d1 = run_ws(M, N, K, 1.0, A, K, B, N, 0.5, C, N, T256, None)
    d2 = run_ws(M, N, K, 1.0, A, K, B, N, 0.5, C, N, T256, None)
    assert np.array_equal(d1.view(np.uint32), d2.view(np.uint32))


def test_unusable_workspace_is_ignored(workspace):
    """A workspace below the size needed, or not 16-byte aligned, leaves the call on the
    one-tile path: the same bits as without a workspace."""
    import torch

    from fp32_gemm_rm_amd import sgemm_rm_op_strided_batched_ws

    M, N, K = 1280, 1536, 300
    A, B, C = make_inputs(M, N, K, K, N, N, "normal", seed=6)
    big = torch.empty(WS_BYTES + 64, dtype=torch.uint8, device="cuda")
    outs = []
    for ptr, nbytes in ((None, 0), (workspace.data_ptr(), WS_BYTES - 4), (big.data_ptr() + 4, WS_BYTES)):
        dA, dB, dC = device(A), device(B), device(C)
        s = torch.cuda.current_stream()
        sgemm_rm_op_strided_batched_ws(0, 0, M, N, K, 1.0, dA.data_ptr(), K, 0, dB.data_ptr(), N, 0, 0.0,
                                       dC.data_ptr(), N, 0, 1, ptr, nbytes, s.cuda_stream, T256)
        s.synchronize()
        outs.append(dC.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))


def test_default_path_4608_full(oracle, workspace):
    """4608^3 (324 tiles of 256^2, 1.27 waves): the default path with a workspace chooses
    stream-K; normal inputs, beta = 1, every output within the bound."""
    from fp32_gemm_rm_amd import sgemm_rm_workspace_size

    M = N = K = 4608
    assert sgemm_rm_workspace_size(M, N, K) == WS_BYTES
    print("[stream-k] 4608^3 default path", flush=True)
    A, B, C = make_inputs(M, N, K, K, N, N, "normal", seed=51, c_init="random")
    out = run_ws(M, N, K, 1.0, A, K, B, N, 1.0, C, N, 0, workspace)
    ref, S = oracle.full(M, N, K, 1.0, A, K, B, N, 1.0, C, N)
    r = assert_within_bound(out.reshape(M, N), ref, S, "4608^3 stream-K")
    print(f"[stream-k] 4608^3 every output, max err/bound {r:.3g}", flush=True)
