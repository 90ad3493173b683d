"""The C-ABI library without a GPU: it loads, exports what the header declares,
and rejects invalid arguments before making any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm_rm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:long\s+long|\w+)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from fp32_gemm_rm_amd import binding

    if not os.path.exists(binding.library_path()):
        pytest.fail("libsgemm_rm.so is not built (run __graft_entry__.build())")
    return binding.load_library()


def test_header_declares_the_entry_points():
    assert _declared_functions() == ["sgemm_cm", "sgemm_cm_strided_batched_ex", "sgemm_cm_strided_batched_ws",
                                     "sgemm_rm", "sgemm_rm_ex", "sgemm_rm_op", "sgemm_rm_op_strided_batched_ex",
                                     "sgemm_rm_op_strided_batched_noalloc", "sgemm_rm_op_strided_batched_ws", "sgemm_rm_plan_tiles", "sgemm_rm_strerror",
                                     "sgemm_rm_strided_batched", "sgemm_rm_strided_batched_ex", "sgemm_rm_version",
                                     "sgemm_rm_workspace_size"]


def test_library_exports_every_declared_symbol(lib):
    from fp32_gemm_rm_amd.binding import EXPORTED_SYMBOLS, library_path

    raw = ctypes.CDLL(library_path())
    for name in _declared_functions():
        assert hasattr(raw, name), name
    assert set(EXPORTED_SYMBOLS) == set(_declared_functions())
    assert lib.sgemm_rm_version() == 400


def test_poison_library_exports_every_declared_symbol(lib):
    """The LDS-poisoning debug build (the GPU tests' check for reads of unwritten LDS) is
    built beside the library and exports the same C ABI."""
    from fp32_gemm_rm_amd.binding import load_poison_library

    poison = load_poison_library()
    for name in _declared_functions():
        assert hasattr(poison, name), name
    assert poison.sgemm_rm_version() == 400
    assert poison.sgemm_rm_plan_tiles(4096, 4096, 4096, 1) == lib.sgemm_rm_plan_tiles(4096, 4096, 4096, 1)


F = 0x1000  # a non-null dummy pointer: never dereferenced, the calls return before any launch


@pytest.mark.parametrize(
    "args,code",
    [
        ((-1, 4, 4, 1.0, F, 4, F, 4, 0.0, F, 4), -1),
        ((4, -1, 4, 1.0, F, 4, F, 4, 0.0, F, 4), -2),
        ((4, 4, -1, 1.0, F, 4, F, 4, 0.0, F, 4), -3),
        ((4, 4, 4, 1.0, None, 4, F, 4, 0.0, F, 4), -5),
        ((4, 4, 4, 1.0, F, 3, F, 4, 0.0, F, 4), -6),
        ((4, 4, 4, 1.0, F, 4, None, 4, 0.0, F, 4), -7),
        ((4, 4, 4, 1.0, F, 4, F, 3, 0.0, F, 4), -8),
        ((4, 4, 4, 1.0, F, 4, F, 4, 0.0, None, 4), -10),
        ((4, 4, 4, 1.0, F, 4, F, 4, 0.0, F, 3), -11),
        ((4, 4, 4, 1.0, F, 4, F, 4, 0.0, F, 0), -11),
        ((4, 4, 4, 1.0, F, 0, F, 4, 0.0, F, 4), -6),
    ],
)
def test_invalid_arguments(lib, args, code):
    assert lib.sgemm_rm(*args, None) == code
    assert lib.sgemm_rm_ex(*args, None, 0) == code


def test_unknown_variant(lib):
    assert lib.sgemm_rm_ex(4, 4, 4, 1.0, F, 4, F, 4, 0.0, F, 4, None, 11) == -13
    assert lib.sgemm_rm_ex(4, 4, 4, 1.0, F, 4, F, 4, 0.0, F, 4, None, -1) == -13


def test_first_invalid_argument_wins(lib):
    assert lib.sgemm_rm(-1, -1, -1, 1.0, None, 0, None, 0, 0.0, None, 0, None) == -1


def test_null_operands_allowed_when_not_read(lib):
    # M == 0 or N == 0: nothing is read or written, nothing is launched
    assert lib.sgemm_rm(0, 5, 5, 1.0, None, 5, None, 5, 0.0, None, 5, None) == 0
    assert lib.sgemm_rm(5, 0, 5, 1.0, None, 5, None, 1, 0.0, None, 1, None) == 0
    # alpha == 0 and beta == 1: C is unchanged, nothing is launched, A and B may be NULL
    assert lib.sgemm_rm(5, 5, 5, 0.0, None, 5, None, 5, 1.0, F, 5, None) == 0
    # K == 0 and beta == 1: likewise
    assert lib.sgemm_rm(5, 5, 0, 1.0, None, 1, None, 5, 1.0, F, 5, None) == 0


def test_strerror(lib):
    from fp32_gemm_rm_amd import sgemm_rm_strerror

    assert sgemm_rm_strerror(0) == "success"
    for code in range(-21, 0):
        assert sgemm_rm_strerror(code) == f"invalid argument {-code}"
    assert sgemm_rm_strerror(-99) == "unknown error code"


def test_binding_raises_on_invalid_arguments(lib):
    """A negative return code (an invalid argument) raises a ValueError, not a RuntimeError."""
    from fp32_gemm_rm_amd import SgemmArgumentError, SgemmError, sgemm_rm, sgemm_rm_plan_tiles

    with pytest.raises(ValueError) as e:
        sgemm_rm(4, 4, 4, 1.0, F, 2, F, 4, 0.0, F, 4)
    assert e.value.code == -6
    assert isinstance(e.value, SgemmArgumentError) and isinstance(e.value, SgemmError)
    assert not isinstance(e.value, RuntimeError)
    with pytest.raises(ValueError) as e:
        sgemm_rm_plan_tiles(4, -2, 4)
    assert e.value.code == -2


def test_binding_raises_runtime_error_on_hip_errors(lib):
    """A positive return code (the hipError_t of a launch) raises a RuntimeError, not a
    ValueError; the message is the HIP runtime's text for the code."""
    from fp32_gemm_rm_amd import SgemmLaunchError, binding

    hip_error_invalid_configuration = 9
    with pytest.raises(RuntimeError) as e:
        binding._check(hip_error_invalid_configuration)
    assert isinstance(e.value, SgemmLaunchError) and not isinstance(e.value, ValueError)
    assert e.value.code == hip_error_invalid_configuration
    assert binding._check(0) == 0


G = 1 << 20  # a batch stride large enough for the 4 x 4 problems below


@pytest.mark.parametrize(
    "args,code",
    [
        ((-1, 4, 4, 1.0, F, 4, G, F, 4, G, 0.0, F, 4, G, 2), -1),
        ((4, -1, 4, 1.0, F, 4, G, F, 4, G, 0.0, F, 4, G, 2), -2),
        ((4, 4, -1, 1.0, F, 4, G, F, 4, G, 0.0, F, 4, G, 2), -3),
        ((4, 4, 4, 1.0, None, 4, G, F, 4, G, 0.0, F, 4, G, 2), -5),
        ((4, 4, 4, 1.0, F, 3, G, F, 4, G, 0.0, F, 4, G, 2), -6),
        ((4, 4, 4, 1.0, F, 4, -1, F, 4, G, 0.0, F, 4, G, 2), -7),
        ((4, 4, 4, 1.0, F, 4, G, None, 4, G, 0.0, F, 4, G, 2), -8),
        ((4, 4, 4, 1.0, F, 4, G, F, 3, G, 0.0, F, 4, G, 2), -9),
        ((4, 4, 4, 1.0, F, 4, G, F, 4, -4, 0.0, F, 4, G, 2), -10),
        ((4, 4, 4, 1.0, F, 4, G, F, 4, G, 0.0, None, 4, G, 2), -12),
        ((4, 4, 4, 1.0, F, 4, G, F, 4, G, 0.0, F, 3, G, 2), -13),
        ((4, 4, 4, 1.0, F, 4, G, F, 4, G, 0.0, F, 4, 15, 2), -14),  # outputs overlap: 3*4+4 = 16 > 15
        ((4, 4, 4, 1.0, F, 4, G, F, 4, G, 0.0, F, 4, -16, 2), -14),
        ((4, 4, 4, 1.0, F, 4, G, F, 4, G, 0.0, F, 4, G, -1), -15),
    ],
)
def test_batched_invalid_arguments(lib, args, code):
    assert lib.sgemm_rm_strided_batched(*args, None) == code
    assert lib.sgemm_rm_strided_batched_ex(*args, None, 0) == code


def test_batched_quick_returns_and_variant(lib):
    # batch == 0, M == 0 or N == 0: nothing launched, NULL buffers allowed
    assert lib.sgemm_rm_strided_batched(4, 4, 4, 1.0, None, 4, 0, None, 4, 0, 0.0, None, 4, 0, 0, None) == 0
    assert lib.sgemm_rm_strided_batched(0, 4, 4, 1.0, None, 4, 0, None, 4, 0, 0.0, None, 4, 0, 3, None) == 0
    # a single entry may use any strideC (nothing can overlap)
    assert lib.sgemm_rm_strided_batched(4, 4, 4, 0.0, None, 4, 0, None, 4, 0, 1.0, F, 4, 0, 1, None) == 0
    assert lib.sgemm_rm_strided_batched_ex(4, 4, 4, 1.0, F, 4, G, F, 4, G, 0.0, F, 4, G, 2, None, 11) == -17


# Transposed and column-major forms.  M = 6, N = 5, K = 3 keep every leading-dimension
# bound distinct.  alpha = 0 with beta = 1 makes a valid call return 0 without a launch.
M6, N5, K3 = 6, 5, 3


def _min_lds(cm, ta, tb):
    """Smallest valid (lda, ldb, ldc) for the stored shapes of op(A) 6 x 3, op(B) 3 x 5, C 6 x 5."""
    a_rows, a_cols = (K3, M6) if ta else (M6, K3)
    b_rows, b_cols = (N5, K3) if tb else (K3, N5)
    if cm:
        return a_rows, b_rows, M6
    return a_cols, b_cols, N5


ORIENTATIONS = [(0, 0), (0, 1), (1, 0), (1, 1)]


@pytest.mark.parametrize("cm", [False, True], ids=["rm", "cm"])
@pytest.mark.parametrize("ta,tb", ORIENTATIONS)
def test_op_leading_dimension_bounds(lib, cm, ta, tb):
    fn = lib.sgemm_cm if cm else lib.sgemm_rm_op
    lda, ldb, ldc = _min_lds(cm, ta, tb)
    assert fn(ta, tb, M6, N5, K3, 0.0, F, lda, F, ldb, 1.0, F, ldc, None) == 0
    assert fn(ta, tb, M6, N5, K3, 0.0, F, lda - 1, F, ldb, 1.0, F, ldc, None) == -8
    assert fn(ta, tb, M6, N5, K3, 0.0, F, lda, F, ldb - 1, 1.0, F, ldc, None) == -10
    assert fn(ta, tb, M6, N5, K3, 0.0, F, lda, F, ldb, 1.0, F, ldc - 1, None) == -13
    bfn = lib.sgemm_cm_strided_batched_ex if cm else lib.sgemm_rm_op_strided_batched_ex
    extent = (N5 - 1) * ldc + M6 if cm else (M6 - 1) * ldc + N5
    ok = (ta, tb, M6, N5, K3, 0.0, F, lda, G, F, ldb, G, 1.0, F, ldc, extent, 3, None, 0)
    assert bfn(*ok) == 0
    assert bfn(*ok[:7], lda - 1, *ok[8:]) == -8
    assert bfn(*ok[:10], ldb - 1, *ok[11:]) == -11
    assert bfn(*ok[:14], ldc - 1, *ok[15:]) == -15
    assert bfn(*ok[:15], extent - 1, *ok[16:]) == -16


@pytest.mark.parametrize("cm", [False, True], ids=["rm", "cm"])
def test_op_invalid_arguments(lib, cm):
    fn = lib.sgemm_cm if cm else lib.sgemm_rm_op
    lda, ldb, ldc = _min_lds(cm, 0, 0)
    ok = [0, 0, M6, N5, K3, 1.0, F, lda, F, ldb, 0.0, F, ldc, None]
    for pos, bad in [(1, 2), (1, -1), (2, 2), (3, -1), (4, -1), (5, -1), (7, None), (9, None), (12, None)]:
        args = list(ok)
        args[pos - 1] = bad
        assert fn(*args) == -pos, (pos, bad)
    bfn = lib.sgemm_cm_strided_batched_ex if cm else lib.sgemm_rm_op_strided_batched_ex
    bok = [0, 0, M6, N5, K3, 1.0, F, lda, G, F, ldb, G, 0.0, F, ldc, G, 2, None, 0]
    for pos, bad in [(1, 3), (2, -1), (3, -1), (4, -1), (5, -1), (7, None), (9, -1), (10, None), (12, -1),
                     (14, None), (16, -1), (17, -1), (19, 11), (19, -1)]:
        args = list(bok)
        args[pos - 1] = bad
        assert bfn(*args) == -pos, (pos, bad)


def test_op_first_invalid_argument_wins(lib):
    assert lib.sgemm_rm_op(7, 7, -1, -1, -1, 1.0, None, 0, None, 0, 0.0, None, 0, None) == -1
    assert lib.sgemm_cm(0, 7, -1, -1, -1, 1.0, None, 0, None, 0, 0.0, None, 0, None) == -2


def test_python_operand_layout():
    """The tensor-level call reads a row-major view as op N and a transposed view as op T
    of the row-major matrix underneath, with that matrix's leading dimension."""
    import torch

    from fp32_gemm_rm_amd.binding import SGEMM_RM_OP_N, SGEMM_RM_OP_T, operand_layout

    base = torch.zeros(7, 9)
    for view, expect in [(base, (9, SGEMM_RM_OP_N)), (base[:, :5], (9, SGEMM_RM_OP_N)),
                         (base.t(), (9, SGEMM_RM_OP_T)), (base[:, :5].t(), (9, SGEMM_RM_OP_T)),
                         (base[:1, :], (9, SGEMM_RM_OP_N)), (base[:, :1], (9, SGEMM_RM_OP_N)),
                         (base[:1, :].t(), (1, SGEMM_RM_OP_N))]:
        assert operand_layout(*view.shape, *view.stride()) == expect, (view.shape, view.stride())
    with pytest.raises(ValueError):
        operand_layout(*base[::2, ::2].shape, *base[::2, ::2].stride())
    with pytest.raises(ValueError):  # overlapping rows
        operand_layout(4, 8, 4, 1)


def test_plan_tiles(lib):
    """The tile plan is a host-side choice: quick returns, argument codes, and the
    configurations the model picks for the benchmark workloads."""
    from fp32_gemm_rm_amd import sgemm_rm_plan_tiles

    assert lib.sgemm_rm_plan_tiles(-1, 4, 4, 1) == -1
    assert lib.sgemm_rm_plan_tiles(4, -1, 4, 1) == -2
    assert lib.sgemm_rm_plan_tiles(4, 4, -1, 1) == -3
    assert lib.sgemm_rm_plan_tiles(4, 4, 4, -1) == -4
    assert lib.sgemm_rm_plan_tiles(0, 4, 4, 1) == 0 and lib.sgemm_rm_plan_tiles(4, 4, 4, 0) == 0
    assert sgemm_rm_plan_tiles(4096, 4096, 4096) == 256
    assert sgemm_rm_plan_tiles(8192, 8192, 8192) == 256
    assert sgemm_rm_plan_tiles(1024, 1024, 1024) == 64
    assert sgemm_rm_plan_tiles(256, 256, 256) == 16  # 256 blocks of 16^2
    assert sgemm_rm_plan_tiles(512, 512, 512) == 32  # 1024 blocks of 16^2 would take four layers
    assert sgemm_rm_plan_tiles(3072, 3072, 3072) == 192  # 256 tiles of 192^2: one whole wave
    # K not a multiple of 16 (no LDS-DMA K loop): 256 x 256 tiles only where they cover the
    # matrix, or leave strips thinner than 16 over one layer of tiles (thin strips after the
    # tiles); wider strips would run as scalar edge tiles
    for n in (4090, 3900):
        assert sgemm_rm_plan_tiles(n, n, n) != 256, n
    assert sgemm_rm_plan_tiles(4096, 4100, 4100) == 256  # 256 tiles and a 4-column thin strip
    assert sgemm_rm_plan_tiles(8200, 8200, 8200) != 256  # thin strips past four layers of tiles
    # K a multiple of 16 (the query assumes 16-byte aligned rows): the direct K loop runs
    # guarded 256 x 256 tiles (4000^3: 892 against 947 us on 128 x 128 tiles), where their
    # layers cost less than the other configurations'
    for M, N, K in ((4000, 4000, 4000), (8000, 8000, 8000), (4096, 4000, 4096), (4096, 4100, 4096)):
        assert sgemm_rm_plan_tiles(M, N, K) == 256, (M, N, K)
    assert sgemm_rm_plan_tiles(3000, 3000, 3008) == 192  # 144 tiles of 256^2 against 256 of 192^2
    assert sgemm_rm_plan_tiles(5000, 5000, 5008) != 256  # 400 tiles: two layers
    assert sgemm_rm_plan_tiles(1000, 1030, 999) == 64  # 6-column thin strip beside 64 x 64 tiles
    assert sgemm_rm_plan_tiles(64, 64, 64, 1024) == 64
    for M, N, K, b in [(1, 1, 1, 1), (5000, 3, 7, 1), (3, 5000, 70000, 1), (65535, 65535, 1, 1000000)]:
        assert sgemm_rm_plan_tiles(M, N, K, b) in (256, 192, 128, 64, 32, 16)


@pytest.mark.parametrize("cm", [False, True], ids=["rm", "cm"])
def test_workspace_call_invalid_arguments(lib, cm):
    """The _ws calls check the workspace pair (positions 18, 19) after batch and before the
    variant (21); everything else as the _ex form, whose checks they share."""
    fn = lib.sgemm_cm_strided_batched_ws if cm else lib.sgemm_rm_op_strided_batched_ws
    lda, ldb, ldc = _min_lds(cm, 0, 0)
    ok = [0, 0, M6, N5, K3, 0.0, F, lda, G, F, ldb, G, 1.0, F, ldc, G, 2, F, 1 << 27, None, 0]
    assert fn(*ok) == 0  # alpha = 0, beta = 1: nothing launched
    for pos, bad in [(1, 2), (3, -1), (8, lda - 1), (17, -1), (18, None), (19, -1), (21, 11), (21, -1)]:
        args = list(ok)
        args[pos - 1] = bad
        assert fn(*args) == -pos, (pos, bad)
    args = list(ok)
    args[17], args[18] = None, 0  # no workspace at all is valid
    assert fn(*args) == 0


def test_workspace_size(lib):
    from fp32_gemm_rm_amd import sgemm_rm_workspace_size

    assert lib.sgemm_rm_workspace_size(-1, 4, 4, 1) == -1
    assert lib.sgemm_rm_workspace_size(4, -1, 4, 1) == -2
    assert lib.sgemm_rm_workspace_size(4, 4, -1, 1) == -3
    assert lib.sgemm_rm_workspace_size(4, 4, 4, -1) == -4
    assert sgemm_rm_workspace_size(0, 4, 4) == 0
    # tiles filling whole waves of 256 workgroups, batches, shapes under one wave: no stream-K
    for M, N, K, b in [(4096, 4096, 4096, 1), (8192, 8192, 8192, 1), (256, 256, 256, 1), (5120, 5120, 5120, 2),
                       (1024, 1024, 1024, 1), (3072, 3072, 3072, 1)]:
        assert sgemm_rm_workspace_size(M, N, K, b) == 0, (M, N, K, b)
    # 4608^3: 324 tiles of 256^2, 1.27 waves: stream-K with two 256 KB slots per workgroup
    assert sgemm_rm_workspace_size(4608, 4608, 4608) == 2 * 256 * 256 * 256 * 4
    # 5120^3 (400 tiles, 1.56 waves): stream-K, modelled (and measured) faster than 192 x 192 tiles
    assert sgemm_rm_workspace_size(5120, 5120, 5120) == 2 * 256 * 256 * 256 * 4
    # 6144^3 (576 tiles, 2.25 waves): 1024 tiles of 192^2 fill four waves and beat stream-K
    assert sgemm_rm_workspace_size(6144, 6144, 6144) == 0
    # stream-K covers full 256 x 256 tiles only
    assert sgemm_rm_workspace_size(4600, 4608, 4608) == 0


def test_noalloc_invalid_arguments_before_any_hip_call(lib):
    """The allocation-free call checks its arguments (positions as the _ex call) before it
    looks up its scratch or launches anything."""
    args = [0, 0, 4, 4, 4, 1.0, F, 4, G, F, 4, G, 0.0, F, 4, G, 2, None, 0]
    fn = lib.sgemm_rm_op_strided_batched_noalloc
    for pos, bad in ((1, 2), (3, -1), (4, -1), (5, -1), (8, 3), (9, -1), (11, 3), (12, -1), (15, 3), (16, 15),
                     (17, -1), (19, 11)):
        a = list(args)
        a[pos - 1] = bad
        assert fn(*a) == -pos, (pos, bad)
    # quick returns touch no scratch and launch nothing
    assert fn(0, 0, 0, 4, 4, 1.0, None, 4, 0, None, 4, 0, 0.0, None, 4, 0, 1, None, 0) == 0
    assert fn(0, 0, 4, 4, 4, 0.0, None, 4, 0, None, 4, 0, 1.0, F, 4, 0, 1, None, 0) == 0


def test_scratch_limit_code(lib):
    from fp32_gemm_rm_amd import binding

    assert binding.SGEMM_RM_SCRATCH_BYTES == 128 << 20
    assert binding.sgemm_rm_strerror(binding.SGEMM_RM_ERR_SCRATCH_LIMIT).startswith("the problem needs more scratch")
    text = open(HEADER).read()
    assert "#define SGEMM_RM_SCRATCH_BYTES (128LL << 20)" in text
    assert "#define SGEMM_RM_ERR_SCRATCH_LIMIT (-100)" in text


# Windows whose tiled launches would need 2^32 or more work-items in one grid: large squares,
# windows a few columns wide and very long ones, and ones just past the banding threshold.
HUGE_WINDOWS = [(65537, 65537, 7), (46341, 46341, 3), (2**31 - 1, 1, 5), (2**31 - 1, 3, 2), (1, 2**31 - 1, 5),
                (3, 2**31 - 1, 2), (100000, 40000, 9), (40000, 100000, 9), (8193, 2**18 + 7, 4)]


@pytest.mark.parametrize("M,N,K", HUGE_WINDOWS)
def test_huge_windows_fit_the_grid_in_every_variant(lib, M, N, K):
    """Host-side check of the launch arithmetic (no GPU here): on a machine without a
    device every call gets as far as its first launch and returns the runtime's
    "no device" code; a grid past the 32-bit work-item count of a dispatch would be
    refused before that with hipErrorInvalidConfiguration (9).  The first launch of a
    banded window is its largest band, so every variant's largest grid is checked.  The
    pointers are dummies that nothing dereferences: no launch can run here."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("needs a machine without a GPU (the calls would launch on dummy pointers)")
    hip_error_invalid_configuration = 9
    for variant in range(11):
        for ta, tb in ((0, 0), (1, 1)):
            lda, ldb = (M if ta else K), (K if tb else N)
            rc = lib.sgemm_rm_op_strided_batched_ex(ta, tb, M, N, K, 1.0, F, lda, 0, F, ldb, 0, 0.0, F, N, 0, 1, None,
                                                    variant)
            assert rc > 0 and rc != hip_error_invalid_configuration, (variant, ta, tb, rc)
