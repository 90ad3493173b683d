"""ctypes binding of the C oracle in ``sgemm_oracle.c`` (test infrastructure only).

The oracle computes the plain definition C = alpha*A*B + beta*C of the sgemmNN
page ("Deep dive into the sgemmNN algorithm", opening section) on row-major
operands with leading dimensions, accumulating in double.  It takes host
float32 buffers and returns float64 results that are never rounded to
float32.  The GPU library is neither imported nor loaded here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "sgemm_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")
GCC_FLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra"]

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def compile_oracle(source: str, out: str) -> str:
    """Compile one oracle source file with gcc (no fast-math, so sums keep their order)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, source], check=True)
    os.replace(tmp, out)
    return out


def build_oracle(force: bool = False) -> str:
    """Build ``liboracle.so`` beside its source when missing or stale (always when ``force``)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE):
        compile_oracle(SOURCE, LIB_PATH)
    return LIB_PATH


def _span_ok(buf, rows: int, cols: int, ld: int, name: str):
    if rows > 0 and cols > 0:
        need = (rows - 1) * ld + cols
        if buf is None or buf.size < need:
            raise ValueError(f"{name}: buffer holds {0 if buf is None else buf.size} floats, needs {need}")


def _as_f32(buf):
    if buf is None:
        return None
    arr = np.ascontiguousarray(np.asarray(buf).reshape(-1))
    if arr.dtype != np.float32:
        raise TypeError("oracle inputs are float32 buffers")
    return arr


def _ptr(arr, typ):
    return None if arr is None else arr.ctypes.data_as(typ)


class Oracle:
    """One loaded oracle library (the real one, or a test's deliberately broken copy)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_sgemm_rm.restype = ctypes.c_int
        lib.oracle_sgemm_rm.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
            _f32p, ctypes.c_long, _f32p, ctypes.c_long, ctypes.c_double, _f32p, ctypes.c_long,
            _f64p, _f64p, ctypes.c_int,
        ]
        lib.oracle_sgemm_rm_entries.restype = ctypes.c_int
        lib.oracle_sgemm_rm_entries.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
            _f32p, ctypes.c_long, _f32p, ctypes.c_long, ctypes.c_double, _f32p, ctypes.c_long,
            _i64p, _i64p, ctypes.c_long, _f64p, _f64p, ctypes.c_int,
        ]
        self.lib = lib
        self.path = path

    def threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def full(self, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, with_absab=True, nthreads=0):
        """Return (C_ref, S), float64 M x N arrays.

        ``C_ref[i, j] = alpha * sum_k A[i*lda+k] * B[k*ldb+j] + beta * C[i*ldc+j]`` and
        ``S[i, j] = sum_k |A[i*lda+k]| * |B[k*ldb+j]|`` (None unless ``with_absab``).
        A, B, C are flat float32 host buffers; C is not read when beta == 0, A and B
        are not read when alpha == 0 or K == 0.
        """
        A, B, C = _as_f32(A), _as_f32(B), _as_f32(C)
        if alpha != 0 and K > 0:
            _span_ok(A, M, K, lda, "A")
            _span_ok(B, K, N, ldb, "B")
        if beta != 0:
            _span_ok(C, M, N, ldc, "C")
        out = np.empty((M, N), dtype=np.float64)
        S = np.empty((M, N), dtype=np.float64) if with_absab else None
        rc = self.lib.oracle_sgemm_rm(
            int(M), int(N), int(K), float(alpha),
            _ptr(A, _f32p), int(lda), _ptr(B, _f32p), int(ldb), float(beta), _ptr(C, _f32p), int(ldc),
            _ptr(out, _f64p), _ptr(S, _f64p), int(nthreads),
        )
        if rc != 0:
            raise ValueError(f"oracle_sgemm_rm returned {rc}")
        return out, S

    def entries(self, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, rows, cols, nthreads=0):
        """Return (values, S), float64 arrays at the entries (rows[e], cols[e])."""
        A, B, C = _as_f32(A), _as_f32(B), _as_f32(C)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        if rows.shape != cols.shape:
            raise ValueError("rows and cols differ in length")
        if alpha != 0 and K > 0:
            _span_ok(A, M, K, lda, "A")
            _span_ok(B, K, N, ldb, "B")
        if beta != 0:
            _span_ok(C, M, N, ldc, "C")
        out = np.empty(rows.size, dtype=np.float64)
        S = np.empty(rows.size, dtype=np.float64)
        rc = self.lib.oracle_sgemm_rm_entries(
            int(M), int(N), int(K), float(alpha),
            _ptr(A, _f32p), int(lda), _ptr(B, _f32p), int(ldb), float(beta), _ptr(C, _f32p), int(ldc),
            _ptr(rows, _i64p), _ptr(cols, _i64p), int(rows.size), _ptr(out, _f64p), _ptr(S, _f64p),
            int(nthreads),
        )
        if rc != 0:
            raise ValueError(f"oracle_sgemm_rm_entries returned {rc}")
        return out, S


_default = None


def default_oracle() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(build_oracle())
    return _default


def oracle_threads() -> int:
    """Threads the oracle's OpenMP loop uses by default."""
    return default_oracle().threads()


def sgemm_rm_ref(*args, **kwargs):
    """``Oracle.full`` on the built oracle."""
    return default_oracle().full(*args, **kwargs)


def sgemm_rm_ref_entries(*args, **kwargs):
    """``Oracle.entries`` on the built oracle."""
    return default_oracle().entries(*args, **kwargs)
