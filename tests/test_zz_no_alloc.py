"""The allocation-free entry point against the call it stands in for, through the C ABI.

sgemm_rm_op_strided_batched_noalloc runs the kernels of
sgemm_rm_op_strided_batched_ws with the library's static scratch as the
workspace, so on the same inputs the two give the same bits.  Two calls in a row
(the second on a smaller problem, which leaves the first call's partial tiles in
the scratch) are each compared with the _ws call given a caller workspace, bit for
bit, and with the oracle: integer inputs (every summation order exact) bit for
bit, random ones within the bound.  The shapes run stream-K and K slices (the
scratch in use) and the one-tile path (scratch unused).
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


def _call(noalloc, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant, ws=None):
    import torch

    from fp32_gemm_rm_amd import sgemm_rm_op_strided_batched_noalloc, sgemm_rm_op_strided_batched_ws

    dA, dB, dC = device(A), device(B), device(C)
    s = torch.cuda.current_stream()
    if noalloc:
        sgemm_rm_op_strided_batched_noalloc(0, 0, M, N, K, alpha, dA.data_ptr(), lda, 0, dB.data_ptr(), ldb, 0,
                                            beta, dC.data_ptr(), ldc, 0, 1, s.cuda_stream, variant)
    else:
        sgemm_rm_op_strided_batched_ws(0, 0, M, N, K, alpha, dA.data_ptr(), lda, 0, dB.data_ptr(), ldb, 0, beta,
                                       dC.data_ptr(), ldc, 0, 1, ws.data_ptr(), ws.numel(), s.cuda_stream, variant)
    s.synchronize()
    return dC.cpu().numpy()


def _integer_case(M, N, K, seed):
    lda, ldb, ldc = K + 4, N + 8, N + 3
    a = integer_matrix(M, K, -4, 4, seed=seed)
    b = integer_matrix(K, N, -4, 4, seed=seed + 1)
    c = integer_matrix(M, N, -4, 4, seed=seed + 2)
    return (M, N, K, lda, ldb, ldc, pad_rows(a, lda, np.nan), pad_rows(b, ldb, np.nan),
            pad_rows(c, ldc, C_PAD_SENTINEL))


@pytest.mark.parametrize("variant", [T256, 0])
def test_noalloc_matches_workspace_call_twice(oracle, variant):
    """Stream-K shapes: 289 tiles of 256^2 (256 one-tile workgroups + 33 stream-K tiles,
    with scalar edge tiles), then a smaller 20-tile product; each call equals the _ws call
    bit for bit and the oracle bit for bit (integer inputs)."""
    import torch

    ws = torch.empty(WS_BYTES, dtype=torch.uint8, device="cuda")
    for M, N, K, seed in ((4352 + 37, 4352 + 19, 40, 31), (1024, 1280, 77, 32)):
        print(f"[noalloc] {M}x{N}x{K} variant {variant}", flush=True)
        M, N, K, lda, ldb, ldc, A, B, C = _integer_case(M, N, K, seed)
        got = _call(True, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, variant)
        want = _call(False, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, variant, ws)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{M}x{N}x{K}: differs from the _ws call"
        ref, _ = oracle.full(M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, with_absab=False)
        bad = np.argwhere(c_window(got, M, N, ldc).astype(np.float64) != ref)
        assert bad.size == 0, f"{M}x{N}x{K}: {len(bad)} mismatches, first at {bad[:3].tolist()}"
        check_padding(got, C, M, N, ldc)


def test_noalloc_default_path_random_twice(oracle):
    """The default path's own stream-K choice at 4608^3 (normal inputs, beta = 1), then a
    smaller product on the one-tile path: each equals the _ws call bit for bit and is within
    the bound of the oracle."""
    import torch

    from fp32_gemm_rm_amd import sgemm_rm_workspace_size

    ws = torch.empty(WS_BYTES, dtype=torch.uint8, device="cuda")
    for M, N, K, seed in ((4608, 4608, 4608, 61), (1000, 1030, 999, 62)):
        print(f"[noalloc] default path {M}x{N}x{K}", flush=True)
        lda, ldb, ldc = K + 3, N + 1, N + 2
        A, B, C = make_inputs(M, N, K, lda, ldb, ldc, "normal", seed=seed, c_init="random")
        got = _call(True, M, N, K, 1.0, A, lda, B, ldb, 1.0, C, ldc, 0)
        want = _call(False, M, N, K, 1.0, A, lda, B, ldb, 1.0, C, ldc, 0, ws)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{M}x{N}x{K}: differs from the _ws call"
        ref, S = oracle.full(M, N, K, 1.0, A, lda, B, ldb, 1.0, C, ldc)
        assert_within_bound(c_window(got, M, N, ldc), ref, S, f"noalloc {M}x{N}x{K}")
        check_padding(got, C, M, N, ldc)
    assert sgemm_rm_workspace_size(4608, 4608, 4608) == WS_BYTES


@pytest.mark.parametrize("variant", [7, 0])  # the 64 configuration forced, the default path
def test_noalloc_k_slices_twice(oracle, variant):
    """K slices (12 tiles x 21 slices, then one tile x 195 slices, whose partial tiles
    overwrite the first call's in the scratch): each call equals the _ws call bit for bit
    and the oracle bit for bit (integer inputs)."""
    import torch

    ws = torch.empty(WS_BYTES, dtype=torch.uint8, device="cuda")
    for M, N, K, seed in ((210, 148, 30000, 41), (64, 64, 100000, 42)):
        print(f"[noalloc] K slices {M}x{N}x{K} variant {variant}", flush=True)
        M, N, K, lda, ldb, ldc, A, B, C = _integer_case(M, N, K, seed)
        got = _call(True, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, variant)
        want = _call(False, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, variant, ws)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{M}x{N}x{K}: differs from the _ws call"
        ref, _ = oracle.full(M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc, with_absab=False)
        bad = np.argwhere(c_window(got, M, N, ldc).astype(np.float64) != ref)
        assert bad.size == 0, f"{M}x{N}x{K}: {len(bad)} mismatches, first at {bad[:3].tolist()}"
        check_padding(got, C, M, N, ldc)
