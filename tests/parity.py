"""Helpers shared by the GPU parity tests: device copies, library calls and the bound.

The acceptance bound for float32 results against the oracle's float64 value is
elementwise ``|C_gpu - C_ref| <= 1e-5 * sum_k |a_ik||b_kj| + 1e-6``, applied as
stated (no alpha or beta factors).
"""
from __future__ import annotations

import numpy as np

REL = 1e-5
ABS = 1e-6


def device(buf):
    import torch

    return torch.from_numpy(np.ascontiguousarray(buf)).to("cuda")


def run_gemm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, variant, stream=None, tensors=None):
    """Run the library on copies of the host buffers; returns the float32 C buffer."""
    import torch

    from fp32_gemm_rm_amd import sgemm_rm_ex

    dA, dB, dC = tensors if tensors is not None else (device(A), device(B), device(C))
    s = stream if stream is not None else torch.cuda.current_stream()
    sgemm_rm_ex(M, N, K, alpha, dA.data_ptr(), lda, dB.data_ptr(), ldb, beta, dC.data_ptr(), ldc,
                s.cuda_stream, variant)
    s.synchronize()
    return dC.cpu().numpy()


def c_window(Cbuf, M, N, ldc):
    return Cbuf.reshape(-1)[: M * ldc].reshape(M, ldc)[:, :N] if M * N else np.zeros((M, N), np.float32)


def check_padding(Cout, Cin, M, N, ldc):
    """Columns N..ldc-1 of C are bit-identical before and after."""
    if ldc > N and M > 0:
        a = Cout.reshape(M, ldc)[:, N:].view(np.uint32)
        b = Cin.reshape(M, ldc)[:, N:].view(np.uint32)
        assert np.array_equal(a, b), "C padding was written"


def assert_within_bound(got, ref, S, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite result"
    err = np.abs(got - ref)
    bound = REL * S + ABS
    ratio = err / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape) if ratio.size else None
    assert np.all(err <= bound), (
        f"{what}: max err/bound {ratio.max():.3g} at {worst}: got {got[worst]!r} ref {ref[worst]!r}"
    )
    return float(ratio.max()) if ratio.size else 0.0


def sample_entries(M, N, seed, n_random=4096):
    """Entries to check on a large output: random ones plus whole rows and columns at
    tile boundaries (multiples of 32, 64 and 128 and the last ones)."""
    rng = np.random.default_rng(seed)
    rows = [rng.integers(0, M, n_random)]
    cols = [rng.integers(0, N, n_random)]
    for r in sorted({0, 63, 64, 127, 128, M // 2, M - 129, M - 1}):
        rows.append(np.full(N, r))
        cols.append(np.arange(N))
    for c in sorted({0, 31, 32, 127, 128, N // 2, N - 1}):
        rows.append(np.arange(M))
        cols.append(np.full(M, c))
    return np.concatenate(rows), np.concatenate(cols)


EDGE_DIMS = [1, 2, 3, 7, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def edge_shapes():
    """40 shapes (the 5 cubes plus random picks) with sides around the tile sizes."""
    rng = np.random.default_rng(2024)
    shapes = {(d, d, d) for d in (1, 17, 64, 129, 257)}
    while len(shapes) < 40:
        shapes.add(tuple(int(x) for x in rng.choice(EDGE_DIMS, 3)))
    return sorted(shapes)
