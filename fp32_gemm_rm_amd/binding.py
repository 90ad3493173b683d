"""ctypes binding of ``libsgemm_rm.so`` (declared in ``include/sgemm_rm.h``).

Argument marshalling only: every step of the GEMM runs in the library's HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  The
library is loaded on first use and its absence is an error: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

SGEMM_RM_VARIANT_AUTO = 0
SGEMM_RM_VARIANT_NAIVE = 1
SGEMM_RM_VARIANT_LDS_TILED = 2
SGEMM_RM_VARIANT_REGBLOCK = 3
SGEMM_RM_VARIANT_MFMA = 4
SGEMM_RM_VARIANT_MFMA_T256 = 5
SGEMM_RM_VARIANT_MFMA_T128 = 6
SGEMM_RM_VARIANT_MFMA_T64 = 7
SGEMM_RM_VARIANT_MFMA_T32 = 8
SGEMM_RM_VARIANT_MFMA_T192 = 9
SGEMM_RM_VARIANT_MFMA_T16 = 10
VARIANTS = {
    "auto": SGEMM_RM_VARIANT_AUTO,
    "naive": SGEMM_RM_VARIANT_NAIVE,
    "lds_tiled": SGEMM_RM_VARIANT_LDS_TILED,
    "regblock": SGEMM_RM_VARIANT_REGBLOCK,
    "mfma": SGEMM_RM_VARIANT_MFMA,
    "mfma_t256": SGEMM_RM_VARIANT_MFMA_T256,
    "mfma_t128": SGEMM_RM_VARIANT_MFMA_T128,
    "mfma_t64": SGEMM_RM_VARIANT_MFMA_T64,
    "mfma_t32": SGEMM_RM_VARIANT_MFMA_T32,
    "mfma_t192": SGEMM_RM_VARIANT_MFMA_T192,
    "mfma_t16": SGEMM_RM_VARIANT_MFMA_T16,
}
#: Forced MFMA tile configurations by tile side.
TILE_VARIANTS = {256: SGEMM_RM_VARIANT_MFMA_T256, 192: SGEMM_RM_VARIANT_MFMA_T192, 128: SGEMM_RM_VARIANT_MFMA_T128,
                 64: SGEMM_RM_VARIANT_MFMA_T64, 32: SGEMM_RM_VARIANT_MFMA_T32, 16: SGEMM_RM_VARIANT_MFMA_T16}

SGEMM_RM_OP_N = 0
SGEMM_RM_OP_T = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libsgemm_rm.so"
_lib = None
_poison_lib = None

#: Names the header declares; the CPU tests check that the library exports each.
EXPORTED_SYMBOLS = ("sgemm_rm", "sgemm_rm_ex", "sgemm_rm_strided_batched", "sgemm_rm_strided_batched_ex",
                    "sgemm_rm_op", "sgemm_rm_op_strided_batched_ex", "sgemm_cm", "sgemm_cm_strided_batched_ex",
                    "sgemm_rm_op_strided_batched_ws", "sgemm_cm_strided_batched_ws", "sgemm_rm_workspace_size",
                    "sgemm_rm_plan_tiles", "sgemm_rm_strerror", "sgemm_rm_version",
                    "sgemm_rm_op_strided_batched_noalloc")
#: Bytes of the library's static device scratch (SGEMM_RM_SCRATCH_BYTES) and the code of a
#: call that would need more (SGEMM_RM_ERR_SCRATCH_LIMIT).
SGEMM_RM_SCRATCH_BYTES = 128 << 20
SGEMM_RM_ERR_SCRATCH_LIMIT = -100


class SgemmError(Exception):
    """A nonzero return code of the library (``code``)."""

    def __init__(self, code: int, message: str):
        super().__init__(f"sgemm_rm error {code}: {message}")
        self.code = code


class SgemmArgumentError(SgemmError, ValueError):
    """A negative return code: argument -code of the call is invalid (checked before any HIP call)."""


class SgemmLaunchError(SgemmError, RuntimeError):
    """A positive return code: the hipError_t of a launch (e.g. hipErrorInvalidConfiguration)."""


def error_for(code: int) -> SgemmError:
    """The exception for a nonzero return code: ValueError for an invalid argument,
    RuntimeError for a HIP error."""
    cls = SgemmArgumentError if code < 0 else SgemmLaunchError
    return cls(int(code), sgemm_rm_strerror(int(code)))


def library_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


def load_library():
    """Load the built library (torch first, so that its HIP runtime is the one in use)."""
    global _lib
    if _lib is None:
        _lib = _load(library_path())
    return _lib


def load_poison_library():
    """The LDS-poisoning debug build of the library (every kernel fills its LDS with NaN
    before use), loaded beside the production one with the same argument types; for tests."""
    global _poison_lib
    if _poison_lib is None:
        _poison_lib = _load(os.path.join(os.path.dirname(library_path()), "libsgemm_rm_poison.so"))
    return _poison_lib


def _load(path):
    import torch  # noqa: F401  (loads torch's HIP runtime before the library binds to one)

    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    args = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.sgemm_rm.argtypes = args
    lib.sgemm_rm.restype = ctypes.c_int
    lib.sgemm_rm_ex.argtypes = args + [ctypes.c_int]
    lib.sgemm_rm_ex.restype = ctypes.c_int
    bargs = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
             ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float,
             ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p]
    lib.sgemm_rm_strided_batched.argtypes = bargs
    lib.sgemm_rm_strided_batched.restype = ctypes.c_int
    lib.sgemm_rm_strided_batched_ex.argtypes = bargs + [ctypes.c_int]
    lib.sgemm_rm_strided_batched_ex.restype = ctypes.c_int
    oargs = [ctypes.c_int, ctypes.c_int] + args
    for name in ("sgemm_rm_op", "sgemm_cm"):
        getattr(lib, name).argtypes = oargs
        getattr(lib, name).restype = ctypes.c_int
    obargs = [ctypes.c_int, ctypes.c_int] + bargs + [ctypes.c_int]
    for name in ("sgemm_rm_op_strided_batched_ex", "sgemm_cm_strided_batched_ex"):
        getattr(lib, name).argtypes = obargs
        getattr(lib, name).restype = ctypes.c_int
    wargs = [ctypes.c_int, ctypes.c_int] + bargs[:-1] + [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p,
                                                       ctypes.c_int]
    for name in ("sgemm_rm_op_strided_batched_ws", "sgemm_cm_strided_batched_ws"):
        getattr(lib, name).argtypes = wargs
        getattr(lib, name).restype = ctypes.c_int
    lib.sgemm_rm_op_strided_batched_noalloc.argtypes = obargs
    lib.sgemm_rm_op_strided_batched_noalloc.restype = ctypes.c_int
    lib.sgemm_rm_workspace_size.argtypes = [ctypes.c_int] * 4
    lib.sgemm_rm_workspace_size.restype = ctypes.c_longlong
    lib.sgemm_rm_plan_tiles.argtypes = [ctypes.c_int] * 4
    lib.sgemm_rm_plan_tiles.restype = ctypes.c_int
    lib.sgemm_rm_strerror.argtypes = [ctypes.c_int]
    lib.sgemm_rm_strerror.restype = ctypes.c_char_p
    lib.sgemm_rm_version.argtypes = []
    lib.sgemm_rm_version.restype = ctypes.c_int
    return lib


def sgemm_rm_op_strided_batched_ws(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                                   strideC, batch, workspace, workspace_bytes, stream=0,
                                   variant=SGEMM_RM_VARIANT_AUTO):
    """The general row-major call with a stream-K workspace (device pointer and bytes)."""
    lib = load_library()
    return _check(lib.sgemm_rm_op_strided_batched_ws(
        int(transA), int(transB), int(M), int(N), int(K), float(alpha), A or None, int(lda), int(strideA),
        B or None, int(ldb), int(strideB), float(beta), C or None, int(ldc), int(strideC), int(batch),
        workspace or None, int(workspace_bytes), stream or None, int(variant)))


def sgemm_cm_strided_batched_ws(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                                strideC, batch, workspace, workspace_bytes, stream=0, variant=SGEMM_RM_VARIANT_AUTO):
    """The column-major form of ``sgemm_rm_op_strided_batched_ws``."""
    lib = load_library()
    return _check(lib.sgemm_cm_strided_batched_ws(
        int(transA), int(transB), int(M), int(N), int(K), float(alpha), A or None, int(lda), int(strideA),
        B or None, int(ldb), int(strideB), float(beta), C or None, int(ldc), int(strideC), int(batch),
        workspace or None, int(workspace_bytes), stream or None, int(variant)))


def sgemm_rm_op_strided_batched_noalloc(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C,
                                        ldc, strideC, batch, stream=0, variant=SGEMM_RM_VARIANT_AUTO):
    """The general row-major call with the library's static scratch as its workspace (no
    allocation; calls that overlap on one GPU race on the scratch)."""
    lib = load_library()
    return _check(lib.sgemm_rm_op_strided_batched_noalloc(
        int(transA), int(transB), int(M), int(N), int(K), float(alpha), A or None, int(lda), int(strideA),
        B or None, int(ldb), int(strideB), float(beta), C or None, int(ldc), int(strideC), int(batch),
        stream or None, int(variant)))


def sgemm_rm_workspace_size(M, N, K, batch=1) -> int:
    """Workspace bytes with which the _ws calls use stream-K for the shape (0: none); host only."""
    code = load_library().sgemm_rm_workspace_size(int(M), int(N), int(K), int(batch))
    if code < 0:
        raise error_for(int(code))
    return int(code)


_workspaces = {}


def _workspace_for(M, N, K, device, stream):
    """(pointer, bytes) of a cached device workspace for the calls on `stream`, or (None, 0)."""
    import torch

    need = sgemm_rm_workspace_size(M, N, K, 1)
    if need == 0:
        return None, 0
    key = (device.index, stream.cuda_stream)
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < need:
        buf = torch.empty(need, dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    return buf.data_ptr(), buf.numel()


def sgemm_rm_plan_tiles(M, N, K, batch=1) -> int:
    """Tile side of the MFMA configuration the library picks for the shape (host only)."""
    code = load_library().sgemm_rm_plan_tiles(int(M), int(N), int(K), int(batch))
    if code < 0:
        raise error_for(code)
    return code


def sgemm_rm_strerror(code: int) -> str:
    return load_library().sgemm_rm_strerror(int(code)).decode()


def _check(code: int) -> int:
    if code != 0:
        raise error_for(code)
    return code


def sgemm_rm(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0):
    """C := alpha*A*B + beta*C on raw device pointers (ints); raises SgemmArgumentError (a ValueError) on an
    invalid argument and SgemmLaunchError (a RuntimeError) on a HIP error."""
    lib = load_library()
    return _check(lib.sgemm_rm(int(M), int(N), int(K), float(alpha), A or None, int(lda), B or None,
                               int(ldb), float(beta), C or None, int(ldc), stream or None))


def sgemm_rm_ex(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0, variant=SGEMM_RM_VARIANT_AUTO):
    """As ``sgemm_rm`` with the kernel family forced; raises SgemmError on failure."""
    lib = load_library()
    return _check(lib.sgemm_rm_ex(int(M), int(N), int(K), float(alpha), A or None, int(lda), B or None,
                                  int(ldb), float(beta), C or None, int(ldc), stream or None, int(variant)))


def sgemm_rm_strided_batched(M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch,
                             stream=0):
    """Strided batch of C_b := alpha*A_b*B_b + beta*C_b on raw device pointers; raises SgemmError."""
    lib = load_library()
    return _check(lib.sgemm_rm_strided_batched(
        int(M), int(N), int(K), float(alpha), A or None, int(lda), int(strideA), B or None, int(ldb),
        int(strideB), float(beta), C or None, int(ldc), int(strideC), int(batch), stream or None))


def sgemm_rm_strided_batched_ex(M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc, strideC, batch,
                                stream=0, variant=SGEMM_RM_VARIANT_AUTO):
    """As ``sgemm_rm_strided_batched`` with the kernel family forced."""
    lib = load_library()
    return _check(lib.sgemm_rm_strided_batched_ex(
        int(M), int(N), int(K), float(alpha), A or None, int(lda), int(strideA), B or None, int(ldb),
        int(strideB), float(beta), C or None, int(ldc), int(strideC), int(batch), stream or None, int(variant)))


def sgemm_rm_op(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0):
    """C := alpha*op(A)*op(B) + beta*C, row-major, on raw device pointers; raises SgemmError."""
    lib = load_library()
    return _check(lib.sgemm_rm_op(int(transA), int(transB), int(M), int(N), int(K), float(alpha), A or None,
                                  int(lda), B or None, int(ldb), float(beta), C or None, int(ldc), stream or None))


def sgemm_rm_op_strided_batched_ex(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                                   strideC, batch, stream=0, variant=SGEMM_RM_VARIANT_AUTO):
    """The general row-major call (operation arguments, strided batch, kernel family)."""
    lib = load_library()
    return _check(lib.sgemm_rm_op_strided_batched_ex(
        int(transA), int(transB), int(M), int(N), int(K), float(alpha), A or None, int(lda), int(strideA),
        B or None, int(ldb), int(strideB), float(beta), C or None, int(ldc), int(strideC), int(batch),
        stream or None, int(variant)))


def sgemm_cm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0):
    """C := alpha*op(A)*op(B) + beta*C, column-major (BLAS), on raw device pointers."""
    lib = load_library()
    return _check(lib.sgemm_cm(int(transA), int(transB), int(M), int(N), int(K), float(alpha), A or None,
                               int(lda), B or None, int(ldb), float(beta), C or None, int(ldc), stream or None))


def sgemm_cm_strided_batched_ex(transA, transB, M, N, K, alpha, A, lda, strideA, B, ldb, strideB, beta, C, ldc,
                                strideC, batch, stream=0, variant=SGEMM_RM_VARIANT_AUTO):
    """Strided batch of column-major problems with the kernel family forced."""
    lib = load_library()
    return _check(lib.sgemm_cm_strided_batched_ex(
        int(transA), int(transB), int(M), int(N), int(K), float(alpha), A or None, int(lda), int(strideA),
        B or None, int(ldb), int(strideB), float(beta), C or None, int(ldc), int(strideC), int(batch),
        stream or None, int(variant)))


def operand_layout(rows, cols, stride0, stride1, name="X"):
    """(ld, op) of a rows x cols view with element strides (stride0, stride1), read as
    op(X): a view with unit column stride is a row-major matrix (op N, ld = stride0);
    one with unit row stride (``X.t()`` of a row-major X) is the transpose of the
    row-major matrix underneath (op T, ld = stride1)."""
    if cols <= 1 or stride1 == 1:
        ld = stride0 if rows > 1 else max(cols, 1)
        if ld < max(cols, 1):
            raise ValueError(f"{name} rows overlap (stride(0) = {ld} < {cols} columns)")
        return ld, SGEMM_RM_OP_N
    if rows <= 1 or stride0 == 1:
        ld = stride1 if cols > 1 else max(rows, 1)
        if ld < max(rows, 1):
            raise ValueError(f"{name} columns overlap (stride(1) = {ld} < {rows} rows)")
        return ld, SGEMM_RM_OP_T
    raise ValueError(f"{name} needs a unit stride along one dimension")


def _device_matrix(t, name):
    import torch

    if t.dtype != torch.float32 or t.dim() != 2 or not t.is_cuda:
        raise TypeError(f"{name} must be a 2-D float32 device tensor")


def _operand_view(t, name):
    """(pointer, ld, op) of a 2-D float32 device tensor read as op(X)."""
    _device_matrix(t, name)
    ld, op = operand_layout(t.shape[0], t.shape[1], t.stride(0), t.stride(1), name)
    return t.data_ptr(), ld, op


def _matrix_view(t, name):
    """(pointer, ld) of a row-major 2-D float32 device tensor view."""
    _device_matrix(t, name)
    ld, op = operand_layout(t.shape[0], t.shape[1], t.stride(0), t.stride(1), name)
    if op != SGEMM_RM_OP_N:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    return t.data_ptr(), ld


def sgemm_batched(A, B, C, alpha=1.0, beta=0.0, variant=SGEMM_RM_VARIANT_AUTO, stream=None):
    """C[b] := alpha*A[b]@B[b] + beta*C[b] in place on 3-D float32 device tensors (row-major
    matrices; stride(0) is the batch stride, stride(1) the leading dimension)."""
    import torch

    if isinstance(variant, str):
        variant = VARIANTS[variant]
    for t, name in ((A, "A"), (B, "B"), (C, "C")):
        if t.dtype != torch.float32 or t.dim() != 3 or not t.is_cuda:
            raise TypeError(f"{name} must be a 3-D float32 device tensor")
    nb, M, K = A.shape
    nb2, K2, N = B.shape
    if K2 != K or nb2 != nb or tuple(C.shape) != (nb, M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    a, lda = _matrix_view(A[0], "A") if nb else (A.data_ptr(), max(K, 1))
    b, ldb = _matrix_view(B[0], "B") if nb else (B.data_ptr(), max(N, 1))
    c, ldc = _matrix_view(C[0], "C") if nb else (C.data_ptr(), max(N, 1))
    s = (stream if stream is not None else torch.cuda.current_stream(C.device)).cuda_stream
    return sgemm_rm_strided_batched_ex(M, N, K, alpha, a, lda, A.stride(0), b, ldb, B.stride(0), beta, c, ldc,
                                       C.stride(0), nb, s, variant)


def sgemm(A, B, C, alpha=1.0, beta=0.0, variant=SGEMM_RM_VARIANT_AUTO, stream=None, workspace=True):
    """C := alpha*A@B + beta*C in place on 2-D float32 device tensors, on torch's current
    stream unless ``stream`` is given.  C is a row-major view (leading dimension =
    stride(0)); A and B may be row-major views or transposed ones (``X.t()`` of a
    row-major X), which run as the transposed-operand forms without a copy.  With
    ``workspace`` the call gets a cached per-stream device workspace where the library's
    cost model chooses stream-K for the shape."""
    import torch

    if isinstance(variant, str):
        variant = VARIANTS[variant]
    M, K = A.shape
    K2, N = B.shape
    if K2 != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    a, lda, ta = _operand_view(A, "A")
    b, ldb, tb = _operand_view(B, "B")
    c, ldc = _matrix_view(C, "C")
    st = stream if stream is not None else torch.cuda.current_stream(C.device)
    ws, ws_bytes = _workspace_for(M, N, K, C.device, st) if workspace else (None, 0)
    return sgemm_rm_op_strided_batched_ws(ta, tb, M, N, K, alpha, a, lda, 0, b, ldb, 0, beta, c, ldc, 0, 1, ws,
                                          ws_bytes, st.cuda_stream, variant)
