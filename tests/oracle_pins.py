"""Pins of the CPU oracle to facts it does not compute itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with something the definition C = alpha*A*B + beta*C
("Deep dive into the sgemmNN algorithm", opening section) or plain
mathematics fixes: exact rational brute force on tiny shapes, the identity,
all-ones, rank-1 outer products, alpha = 0, beta = 0, integer-valued inputs
(against numpy's exact int64 product) and strided inputs (against numpy's
float64 product).  Every pin checks both oracle entry points (the full result
and the sampled entries).  The same functions run against deliberately broken
copies of the oracle to show that each plausible mistake fails one of them.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from fp32_gemm_rm_amd.workloads import C_PAD_SENTINEL, integer_matrix, make_inputs, pad_rows

U53 = 2.0 ** -53


def _all_entries(M, N):
    r, c = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    return r.reshape(-1), c.reshape(-1)


def both(orc, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    """Full result and the entries path at every (i, j); both as M x N arrays."""
    full, S = orc.full(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    if M * N == 0:
        return [(full, S)]
    r, c = _all_entries(M, N)
    ev, es = orc.entries(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, r, c)
    return [(full, S), (ev.reshape(M, N), es.reshape(M, N))]


def exact_reference(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
    """Exact rational result and exact sum |a||b| from the floats' exact values."""
    fa, fb = Fraction(float(alpha)), Fraction(float(beta))
    out = [[Fraction(0)] * N for _ in range(M)]
    absab = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            sa = Fraction(0)
            if alpha != 0:
                for k in range(K):
                    a = Fraction(float(A[i * lda + k]))
                    b = Fraction(float(B[k * ldb + j]))
                    s += a * b
                    sa += abs(a) * abs(b)
            v = fa * s
            if beta != 0:
                v += fb * Fraction(float(C[i * ldc + j]))
            out[i][j] = v
            absab[i][j] = sa
    return out, absab


TINY_SHAPES = [(1, 1, 1), (2, 3, 4), (3, 2, 5), (4, 4, 4), (5, 7, 3), (7, 5, 8), (8, 8, 2), (1, 8, 7),
               (7, 1, 1), (3, 4, 0)]
SCALARS = [0.0, 1.0, -1.0, 0.5, 1.5, -0.5, 0.3]


def pin_brute_force(orc):
    """Exact rational arithmetic on tiny shapes with padded leading dimensions."""
    rng = np.random.default_rng(1234)
    for t, (M, N, K) in enumerate(TINY_SHAPES):
        alpha = float(np.float32(SCALARS[t % len(SCALARS)]))
        beta = float(np.float32(SCALARS[(3 * t + 1) % len(SCALARS)]))
        lda, ldb, ldc = K + 1 + t % 3, N + 2, N + 1 + t % 2
        A, B, C = make_inputs(M, N, K, lda, ldb, ldc, "uniform", seed=100 + t, c_init="random")
        # widen the exponent range a little so that a dropped or doubled term shows
        A = A * np.float32(rng.choice([0.25, 1.0, 4.0]))
        exact, exact_abs = exact_reference(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
        for got, S in both(orc, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc):
            for i in range(M):
                for j in range(N):
                    e = exact[i][j]
                    scale = abs(alpha) * float(exact_abs[i][j]) + abs(beta) * abs(float(C[i * ldc + j]))
                    tol = (K + 3) * U53 * scale
                    assert np.isfinite(got[i, j]), ("non-finite", M, N, K, i, j)
                    err = abs(Fraction(float(got[i, j])) - e)
                    assert float(err) <= tol, (M, N, K, alpha, beta, i, j, float(got[i, j]), float(e))
                    assert np.isfinite(S[i, j]), ("non-finite S", M, N, K, i, j)
                    serr = abs(Fraction(float(S[i, j])) - exact_abs[i][j])
                    assert float(serr) <= (K + 1) * U53 * float(exact_abs[i][j]), ("S", M, N, K, i, j)


def pin_identity(orc):
    """A = I gives C = B exactly; B = I gives C = A exactly (alpha = 1, beta = 0)."""
    M = K = 6
    N = 9
    lda, ldb, ldc = 8, 11, 10
    eye = pad_rows(np.eye(M, K, dtype=np.float32), lda, np.nan)
    _, B, C = make_inputs(M, N, K, lda, ldb, ldc, "normal", seed=7, c_init="nan")
    for got, _ in both(orc, M, N, K, 1.0, eye, lda, B, ldb, 0.0, C, ldc):
        np.testing.assert_array_equal(got, B.reshape(K, ldb)[:, :N].astype(np.float64))
    M, K, N = 9, 5, 5
    lda, ldb, ldc = 7, 6, 5
    A, _, C = make_inputs(M, N, K, lda, ldb, ldc, "normal", seed=8, c_init="nan")
    eye = pad_rows(np.eye(K, N, dtype=np.float32), ldb, np.nan)
    for got, _ in both(orc, M, N, K, 1.0, A, lda, eye, ldb, 0.0, C, ldc):
        np.testing.assert_array_equal(got, A.reshape(M, lda)[:, :K].astype(np.float64))


def pin_all_ones(orc):
    """A = B = 1 gives K everywhere; with alpha = 1.5, beta = -0.5, C = 1 it gives 1.5K - 0.5."""
    for (M, N, K) in [(3, 5, 7), (4, 2, 33), (1, 1, 100)]:
        lda, ldb, ldc = K + 2, N + 3, N + 1
        A = pad_rows(np.ones((M, K), np.float32), lda, np.nan)
        B = pad_rows(np.ones((K, N), np.float32), ldb, np.nan)
        C0 = pad_rows(np.ones((M, N), np.float32), ldc, C_PAD_SENTINEL)
        for got, S in both(orc, M, N, K, 1.0, A, lda, B, ldb, 0.0, C0, ldc):
            np.testing.assert_array_equal(got, np.full((M, N), float(K)))
            np.testing.assert_array_equal(S, np.full((M, N), float(K)))
        for got, _ in both(orc, M, N, K, 1.5, A, lda, B, ldb, -0.5, C0, ldc):
            np.testing.assert_array_equal(got, np.full((M, N), 1.5 * K - 0.5))


def pin_rank_one(orc):
    """K = 1 gives the outer product a_i * b_j exactly (exact in double)."""
    M, N, K = 7, 6, 1
    lda, ldb, ldc = 3, 9, 8
    A, B, C = make_inputs(M, N, K, lda, ldb, ldc, "normal", seed=11, c_init="nan")
    a = A.reshape(M, lda)[:, 0].astype(np.float64)
    b = B.reshape(K, ldb)[0, :N].astype(np.float64)
    for got, S in both(orc, M, N, K, 1.0, A, lda, B, ldb, 0.0, C, ldc):
        np.testing.assert_array_equal(got, np.outer(a, b))
        np.testing.assert_array_equal(S, np.abs(np.outer(a, b)))
    # A(i,k) = u_i, B(k,j) = v_j with powers of two: C = K u_i v_j exactly for any K
    M, N, K = 5, 4, 37
    lda, ldb, ldc = K, N, N
    u = np.array([0.5, -1.0, 2.0, -0.5, 1.0], np.float32)
    v = np.array([-2.0, 0.5, 1.0, -1.0], np.float32)
    A = np.repeat(u[:, None], K, axis=1).reshape(-1)
    B = np.repeat(v[None, :], K, axis=0).reshape(-1)
    for got, _ in both(orc, M, N, K, 1.0, A, lda, B, ldb, 0.0, None, ldc):
        np.testing.assert_array_equal(got, K * np.outer(u, v).astype(np.float64))


def pin_alpha_zero(orc):
    """alpha = 0 returns beta * C and never reads A or B (they hold NaN)."""
    M, N, K = 5, 6, 4
    lda, ldb, ldc = 4, 7, 9
    A = np.full(M * lda, np.nan, np.float32)
    B = np.full(K * ldb, np.nan, np.float32)
    _, _, C = make_inputs(M, N, K, lda, ldb, ldc, "uniform", seed=12, c_init="random")
    c = C.reshape(M, ldc)[:, :N].astype(np.float64)
    for got, _ in both(orc, M, N, K, 0.0, A, lda, B, ldb, -0.5, C, ldc):
        np.testing.assert_array_equal(got, -0.5 * c)
    # K = 0 is the same case
    for got, _ in both(orc, M, N, 0, 1.0, A, lda, B, ldb, 1.5, C, ldc):
        np.testing.assert_array_equal(got, 1.5 * c)


def pin_beta_zero(orc):
    """beta = 0 never reads C (it holds NaN): the result is finite and equals alpha*A*B."""
    M, N, K = 6, 5, 7
    lda, ldb, ldc = 9, 5, 6
    A, B, C = make_inputs(M, N, K, lda, ldb, ldc, "uniform", seed=13, c_init="nan")
    exact, _ = exact_reference(M, N, K, 1.5, A, lda, B, ldb, 0.0, C, ldc)
    for got, _ in both(orc, M, N, K, 1.5, A, lda, B, ldb, 0.0, C, ldc):
        assert np.all(np.isfinite(got))
        for i in range(M):
            for j in range(N):
                assert abs(Fraction(float(got[i, j])) - exact[i][j]) <= (K + 3) * U53 * 1.5 * K


def pin_integer_exact(orc):
    """Integer-valued inputs: every partial sum is an integer, so the result equals
    numpy's int64 product exactly (also with alpha = 2, beta = -1)."""
    M, N, K = 37, 29, 41
    lda, ldb, ldc = 45, 33, 31
    a = integer_matrix(M, K, -4, 4, seed=21)
    b = integer_matrix(K, N, -4, 4, seed=22)
    c = integer_matrix(M, N, -9, 9, seed=23)
    A, B, C = pad_rows(a, lda, np.nan), pad_rows(b, ldb, np.nan), pad_rows(c, ldc, C_PAD_SENTINEL)
    ref = a.astype(np.int64) @ b.astype(np.int64)
    for got, S in both(orc, M, N, K, 1.0, A, lda, B, ldb, 0.0, C, ldc):
        np.testing.assert_array_equal(got, ref.astype(np.float64))
        np.testing.assert_array_equal(S, (np.abs(a).astype(np.int64) @ np.abs(b).astype(np.int64)))
    ref2 = 2 * ref - c.astype(np.int64)
    for got, _ in both(orc, M, N, K, 2.0, A, lda, B, ldb, -1.0, C, ldc):
        np.testing.assert_array_equal(got, ref2.astype(np.float64))


def pin_strided_float64(orc):
    """Random non-square strided inputs against numpy's float64 product of the views."""
    M, N, K = 23, 17, 31
    lda, ldb, ldc = 36, 20, 19
    A, B, C = make_inputs(M, N, K, lda, ldb, ldc, "normal", seed=31, c_init="random")
    a = A.reshape(M, lda)[:, :K].astype(np.float64)
    b = B.reshape(K, ldb)[:, :N].astype(np.float64)
    c = C.reshape(M, ldc)[:, :N].astype(np.float64)
    ref = 1.5 * (a @ b) - 0.5 * c
    bound = 1.5 * (np.abs(a) @ np.abs(b)) + 0.5 * np.abs(c)
    for got, S in both(orc, M, N, K, 1.5, A, lda, B, ldb, -0.5, C, ldc):
        assert np.all(np.abs(got - ref) <= 4 * (K + 3) * U53 * bound)
        assert np.all(np.abs(S - np.abs(a) @ np.abs(b)) <= 4 * (K + 1) * U53 * S)


ALL_PINS = [pin_brute_force, pin_identity, pin_all_ones, pin_rank_one, pin_alpha_zero, pin_beta_zero,
            pin_integer_exact, pin_strided_float64]
