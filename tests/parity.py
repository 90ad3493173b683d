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


def assert_within_bound(got, ref, S, what="", rows_per_block=1024):
    """Every element within the bound; returns the largest err/bound.  Large outputs are
    compared in blocks of rows, so that the float64 temporaries stay small."""
    got = np.asarray(got)
    if got.ndim < 2 or got.shape[0] <= rows_per_block:
        return _within_bound_block(got, ref, S, what, 0)
    worst = 0.0
    for r0 in range(0, got.shape[0], rows_per_block):
        sl = slice(r0, r0 + rows_per_block)
        worst = max(worst, _within_bound_block(got[sl], ref[sl], S[sl], what, r0))
    return worst


def _within_bound_block(got, ref, S, what, row0):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite result (rows from {row0})"
    err = np.abs(got - ref)
    bound = REL * S + ABS
    ratio = err / bound
    if ratio.size == 0:
        return 0.0
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    at = (worst[0] + row0, *worst[1:]) if ratio.ndim > 1 else worst
    assert np.all(err <= bound), (
        f"{what}: max err/bound {ratio.max():.3g} at {at}: got {got[worst]!r} ref {ref[worst]!r}"
    )
    return float(ratio.max())


def assert_ieee_equal(got, ref, what=""):
    """float32 results against the oracle's float64 ones where both must agree exactly,
    non-finite values included: the same NaN positions, the same +Inf and -Inf positions,
    and equal finite values (zeros compared by value)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    for name, f in (("NaN", np.isnan), ("+Inf", np.isposinf), ("-Inf", np.isneginf)):
        bad = np.argwhere(f(got) != f(ref))
        assert bad.size == 0, f"{what}: {len(bad)} {name} positions differ, first at {bad[:3].tolist()}"
    fin = np.isfinite(ref)
    bad = np.argwhere(fin & (got != ref))
    assert bad.size == 0, f"{what}: {len(bad)} finite values differ, first at {bad[:3].tolist()}"


EDGE_DIMS = [1, 2, 3, 7, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def edge_shapes():
    """40 shapes (the 5 cubes plus random picks) with sides around the tile sizes."""
    rng = np.random.default_rng(2024)
    shapes = {(d, d, d) for d in (1, 17, 64, 129, 257)}
    while len(shapes) < 40:
        shapes.add(tuple(int(x) for x in rng.choice(EDGE_DIMS, 3)))
    return sorted(shapes)
