"""The library from a plain C program (tests/c_client/sgemm_client.c): HIP runtime
buffers, no PyTorch, the C ABI as declared in include/sgemm_rm.h.  The client's integer
inputs come from fixed formulas, rebuilt here for the oracle; the result must match bit
for bit, with the padding of C untouched."""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "probes", "bin", "sgemm_client")

pytestmark = pytest.mark.gpu


def inputs(M, N, K, lda, ldb, ldc):
    def fill(rows, cols, ld, f):
        r, c = np.meshgrid(np.arange(rows), np.arange(ld), indexing="ij")
        return np.where(c < cols, f(r, c) % 9 - 4, -7).astype(np.float32).reshape(-1)

    A = fill(M, K, lda, lambda r, c: 7 * r + 3 * c)
    B = fill(K, N, ldb, lambda r, c: 5 * r + 2 * c + 1)
    C = fill(M, N, ldc, lambda r, c: r + 4 * c + 2)
    return A, B, C


@pytest.mark.parametrize(
    "M,N,K,lda,ldb,ldc,alpha,beta,variant",
    [
        (300, 257, 129, 131, 260, 259, 2.0, -1.0, 0),
        (1024, 1024, 300, 300, 1024, 1030, 1.0, 1.0, 4),
        (200, 150, 77, 80, 150, 151, 0.5, 0.0, 3),
        (64, 96, 33, 33, 96, 96, -1.0, 0.5, 1),
    ],
)
def test_c_client(oracle, tmp_path, M, N, K, lda, ldb, ldc, alpha, beta, variant):
    if not os.path.exists(CLIENT):
        pytest.fail("the C client is not built (run __graft_entry__.build())")
    out = tmp_path / "c.bin"
    args = [CLIENT, *map(str, (M, N, K, lda, ldb, ldc, alpha, beta, variant)), str(out)]
    print("[c-client]", " ".join(args[1:-1]), flush=True)
    proc = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert proc.returncode == 0, proc.stdout + proc.stderr
    got = np.fromfile(out, dtype=np.float32)
    A, B, C = inputs(M, N, K, lda, ldb, ldc)
    ref, _ = oracle.full(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)
    win = got.reshape(M, ldc)
    np.testing.assert_array_equal(win[:, :N].astype(np.float64), ref)
    assert np.array_equal(win[:, N:].view(np.uint32), C.reshape(M, ldc)[:, N:].view(np.uint32))
