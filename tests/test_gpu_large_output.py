"""Outputs of more than 2^32 elements (65537 x 65537, a 17.2 GB C built on the device).

A dispatch counts its work-items in 32 bits per grid dimension.  The
one-thread-per-element kernels (naive, and the C := beta*C pass that alpha == 0
or K == 0 runs in every variant) stride over a capped grid, and the tiled
families run such a window as bands of rows launched one after another (the
host-side arithmetic of every variant's grids is checked on the CPU by
tests/test_abi.py).  The inputs follow closed forms whose every output is exact in float32, so the
whole output is checked on the device chunk by chunk: beta * C for alpha = 0
(special case of the definition with the product term absent), and
K * u_i * v_j for A(i, k) = u_i, B(k, j) = v_j (the rank-1 structure: every
partial sum is an integer), plus sampled rows next to the band seam against
the oracle.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

M = N = 65537  # M * N = 4295098369 > 2^32
CHUNK = 4096


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp32_gemm_rm_amd import load_library

    load_library()
    assert M * N > 2**32
    yield
    torch.cuda.empty_cache()


def _release():
    import torch

    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("variant", [0, 1, 2])  # auto, naive, LDS-tiled: the scale pass is the same for all
def test_alpha_zero_scales_whole_window(variant):
    import torch

    from fp32_gemm_rm_amd import sgemm_rm_ex

    print(f"[large] alpha = 0, variant {variant}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(5)
    c8 = torch.randint(-3, 4, (M * N,), generator=gen, device="cuda", dtype=torch.int8)
    C = c8.to(torch.float32)
    s = torch.cuda.current_stream()
    # beta = -0.5 (exact on integers); A and B are not read and may be NULL
    sgemm_rm_ex(M, N, 7, 0.0, None, 7, None, N, -0.5, C.data_ptr(), N, s.cuda_stream, variant)
    s.synchronize()
    for r0 in range(0, M * N, CHUNK * N):
        r1 = min(r0 + CHUNK * N, M * N)
        assert torch.equal(C[r0:r1], c8[r0:r1].to(torch.float32) * -0.5), f"elements {r0}..{r1}"
    # beta = 0: zeros everywhere, C not read (NaN before the call)
    C.fill_(float("nan"))
    sgemm_rm_ex(M, N, 0, 1.0, None, 1, None, N, 0.0, C.data_ptr(), N, s.cuda_stream, variant)
    s.synchronize()
    for r0 in range(0, M * N, CHUNK * N):
        r1 = min(r0 + CHUNK * N, M * N)
        assert int(torch.count_nonzero(C[r0:r1])) == 0 and not bool(torch.isnan(C[r0:r1]).any())
    del C, c8
    _release()


# auto, naive, LDS-tiled, register-blocked, and the 64 and 16 MFMA configurations forced (the
# 16 one runs 512 threads per 16 x 16 block: the most work-items per output of any launcher)
@pytest.mark.parametrize("variant", [0, 1, 2, 3, 7, 10])
def test_rank_one_structure_whole_window(oracle, variant):
    """A(i, k) = u_i and B(k, j) = v_j with small integers, K = 3: C = 3 u_i v_j exactly
    at every one of the 4.3e9 outputs (beta = 0 with C NaN before the call)."""
    import torch

    from fp32_gemm_rm_amd import sgemm_rm_ex

    K = 3
    print(f"[large] rank-1 structure, variant {variant}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(6)
    u = torch.randint(-4, 5, (M,), generator=gen, device="cuda").to(torch.float32)
    v = torch.randint(-4, 5, (N,), generator=gen, device="cuda").to(torch.float32)
    A = u[:, None].expand(M, K).contiguous()
    B = v[None, :].expand(K, N).contiguous()
    C = torch.full((M, N), float("nan"), device="cuda")
    s = torch.cuda.current_stream()
    sgemm_rm_ex(M, N, K, 1.0, A.data_ptr(), K, B.data_ptr(), N, 0.0, C.data_ptr(), N, s.cuda_stream, variant)
    s.synchronize()
    for r0 in range(0, M, CHUNK):
        r1 = min(r0 + CHUNK, M)
        want = K * torch.outer(u[r0:r1], v)
        assert torch.equal(C[r0:r1], want), f"rows {r0}..{r1}"
    # rows around the seams of the row bands (bands of 32256 rows: 42 x 768, the most whose
    # 16-row-rounded count times ceil(N / 16) = 4097 stays below 2^27) and the last row,
    # against the oracle, bit for bit
    rows = np.array([0, 32255, 32256, 32257, 64511, 64512, 64513, M - 1])
    a_rows = A[torch.from_numpy(rows).cuda()].cpu().numpy().reshape(-1)
    b = B.cpu().numpy().reshape(-1)
    ref, _ = oracle.full(len(rows), N, K, 1.0, a_rows, K, b, N, 0.0, None, N, with_absab=False)
    got = C[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(got, ref)
    del A, B, C
    _release()
