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
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from fp32_gemm_rm_amd import binding

    if not os.path.exists(binding.library_path()):
        pytest.fail("libsgemm_rm.so is not built (run __graft_entry__.build())")
    return binding.load_library()


def test_header_declares_the_entry_points():
    assert _declared_functions() == ["sgemm_rm", "sgemm_rm_ex", "sgemm_rm_strerror", "sgemm_rm_strided_batched",
                                     "sgemm_rm_strided_batched_ex", "sgemm_rm_version"]


def test_library_exports_every_declared_symbol(lib):
    from fp32_gemm_rm_amd.binding import EXPORTED_SYMBOLS, library_path

    raw = ctypes.CDLL(library_path())
    for name in _declared_functions():
        assert hasattr(raw, name), name
    assert set(EXPORTED_SYMBOLS) == set(_declared_functions())
    assert lib.sgemm_rm_version() == 200


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
    assert lib.sgemm_rm_ex(4, 4, 4, 1.0, F, 4, F, 4, 0.0, F, 4, None, 9) == -13
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
    for code in range(-17, 0):
        assert sgemm_rm_strerror(code) == f"invalid argument {-code}"
    assert sgemm_rm_strerror(-99) == "unknown error code"


def test_binding_raises_on_invalid_arguments(lib):
    from fp32_gemm_rm_amd import SgemmError, sgemm_rm

    with pytest.raises(SgemmError) as e:
        sgemm_rm(4, 4, 4, 1.0, F, 2, F, 4, 0.0, F, 4)
    assert e.value.code == -6


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
    assert lib.sgemm_rm_strided_batched_ex(4, 4, 4, 1.0, F, 4, G, F, 4, G, 0.0, F, 4, G, 2, None, 7) == -17
