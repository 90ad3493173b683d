"""The CPU oracle against its pins, and the pins against broken oracles.

CPU only.  The pins (``oracle_pins.py``) tie the oracle to exact rational
arithmetic, closed forms and numpy's integer / float64 products.  The mutation
test compiles copies of ``oracle/sgemm_oracle.c`` with one plausible mistake
planted in each (a dropped term, a wrong sign, a transposed operand, an
ignored leading dimension, a dropped k) and requires every copy to fail at
least one pin.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import compile_oracle
from oracle.oracle import SOURCE

from . import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle, pin):
    pin(oracle)


def test_oracle_entries_match_full(oracle):
    from fp32_gemm_rm_amd.workloads import make_inputs

    M, N, K, lda, ldb, ldc = 40, 33, 57, 60, 35, 34
    A, B, C = make_inputs(M, N, K, lda, ldb, ldc, "uniform", seed=5, c_init="random")
    full, S = oracle.full(M, N, K, 1.5, A, lda, B, ldb, -0.5, C, ldc)
    rng = np.random.default_rng(0)
    r = rng.integers(0, M, 200)
    c = rng.integers(0, N, 200)
    ev, es = oracle.entries(M, N, K, 1.5, A, lda, B, ldb, -0.5, C, ldc, r, c)
    np.testing.assert_array_equal(ev, full[r, c])
    np.testing.assert_array_equal(es, S[r, c])


def test_oracle_rejects_bad_sizes(oracle):
    with pytest.raises(ValueError):
        oracle.entries(2, 2, 2, 1.0, np.zeros(4, np.float32), 2, np.zeros(4, np.float32), 2, 0.0, None,
                       2, [2], [0])
    with pytest.raises(ValueError):
        oracle.full(3, 3, 3, 1.0, np.zeros(4, np.float32), 3, np.zeros(9, np.float32), 3, 0.0, None, 3)


def test_oracle_thread_count_invariant(oracle):
    """Rows are independent: 1 thread and many threads give bit-identical results."""
    from fp32_gemm_rm_amd.workloads import make_inputs

    M, N, K = 64, 48, 80
    A, B, C = make_inputs(M, N, K, K, N, N, "normal", seed=6, c_init="random")
    one, _ = oracle.full(M, N, K, 1.0, A, K, B, N, 1.0, C, N, nthreads=1)
    many, _ = oracle.full(M, N, K, 1.0, A, K, B, N, 1.0, C, N, nthreads=4)
    np.testing.assert_array_equal(one, many)


# (name, [(old, new), ...]); every "old" must occur in the source.
MUTANTS = [
    ("beta_term_dropped", [("if (beta != 0.0) v += beta *", "if (0) v += beta *")]),
    ("beta_sign_flipped", [("v += beta *", "v -= beta *")]),
    ("alpha_dropped", [("product ? alpha * acc[j]", "product ? acc[j]"),
                       ("product ? alpha * s", "product ? s")]),
    ("last_k_dropped", [("for (int k = 0; k < K; ++k)", "for (int k = 0; k + 1 < K; ++k)")]),
    ("lda_ignored", [("(size_t)i * (size_t)lda", "(size_t)i * (size_t)K"),
                     ("i * (size_t)lda + k", "i * (size_t)K + k")]),
    ("ldc_ignored", [("(size_t)i * (size_t)ldc + j", "(size_t)i * (size_t)N + j"),
                     ("i * (size_t)ldc + j", "i * (size_t)N + j")]),
    ("B_transposed", [("acc[j] += a * (double)b_row[j]",
                       "acc[j] += a * (double)B[(size_t)j * (size_t)ldb + k]"),
                      ("const double b = (double)B[(size_t)k * (size_t)ldb + j]",
                       "const double b = (double)B[(size_t)j * (size_t)ldb + k]")]),
    ("absab_signed", [("absab[j] += fabs(a) * fabs((double)b_row[j])", "absab[j] += a * (double)b_row[j]"),
                      ("sa += fabs(a) * fabs(b)", "sa += a * b")]),
]

_RUNNER = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
from oracle import Oracle
from tests import oracle_pins
orc = Oracle(sys.argv[2])
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(orc)
    except AssertionError:
        failed.append(pin.__name__)
print(json.dumps(failed))
"""


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, edits):
    src = open(SOURCE).read()
    for old, new in edits:
        assert old in src, f"mutation anchor {old!r} not in oracle source"
        src = src.replace(old, new)
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(src)
    lib = compile_oracle(str(path), str(tmp_path / f"liboracle_{name}.so"))
    proc = subprocess.run([sys.executable, "-c", _RUNNER, ROOT, lib], capture_output=True, text=True,
                          timeout=300)
    if proc.returncode < 0:
        # killed by a signal (e.g. an out-of-bounds read in the broken copy): exposed as well
        return
    assert proc.returncode == 0, proc.stderr[-2000:]
    failed = json.loads(proc.stdout.strip().splitlines()[-1])
    assert failed, f"no pin caught the planted mistake {name}"
