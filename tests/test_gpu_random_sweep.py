"""Seeded random parity sweep over the whole call surface, through the C ABI.

Each case draws a shape (1 to 700 per side), a kernel family or forced MFMA tile
configuration, transpose flags, row- or column-major storage, padded leading
dimensions, a batch with gaps between entries, alpha and beta from a set that includes
the special values 0 and 1, and whether a stream-K workspace is passed.  Inputs are
integers in [-4, 4], so every summation order is exact and the result must equal the
oracle's bit for bit; C padding and the gaps between batch entries must be untouched.
"""
import numpy as np
import pytest

from fp32_gemm_rm_amd.workloads import C_PAD_SENTINEL, integer_matrix, pad_rows

from .parity import device

pytestmark = pytest.mark.gpu

# auto, naive, lds_tiled, regblock, mfma, mfma with tiles 256/128/64/32/192/16
VARIANTS = [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10]
ALPHAS = [1.0, -1.0, 2.0, 0.5, 0.0]
BETAS = [0.0, 1.0, -1.0, 0.5]
WS_BYTES = 2 * 256 * 256 * 256 * 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp32_gemm_rm_amd import load_library

    load_library()


def stored(mat, trans, cm):
    """The array the call reads for logical `mat`, as a dense rows x cols row-major array."""
    s = mat.T if trans else mat
    return np.ascontiguousarray(s.T if cm else s)


def draw_case(rng):
    dims = [int(rng.choice([rng.integers(1, 80), rng.integers(60, 300), rng.integers(250, 700)])) for _ in range(3)]
    M, N, K = dims
    return dict(M=M, N=N, K=K, variant=int(rng.choice(VARIANTS)), ta=int(rng.integers(0, 2)),
                tb=int(rng.integers(0, 2)), cm=bool(rng.integers(0, 2)), batch=int(rng.choice([1, 1, 1, 2, 3])),
                pads=[int(x) for x in rng.integers(0, 6, 3)], alpha=float(rng.choice(ALPHAS)),
                beta=float(rng.choice(BETAS)), ws=bool(rng.integers(0, 2)))


def run_case(oracle, case, seed, ws_tensor):
    import torch

    from fp32_gemm_rm_amd import sgemm_cm_strided_batched_ws, sgemm_rm_op_strided_batched_ws

    M, N, K, batch = case["M"], case["N"], case["K"], case["batch"]
    ta, tb, cm = case["ta"], case["tb"], case["cm"]
    a = [integer_matrix(M, K, -4, 4, seed=seed * 10 + b) for b in range(batch)]
    bm = [integer_matrix(K, N, -4, 4, seed=seed * 10 + 5 + b) for b in range(batch)]
    c = [integer_matrix(M, N, -4, 4, seed=seed * 10 + 8 + b) for b in range(batch)]
    sa, sb, sc = stored(a[0], ta, cm), stored(bm[0], tb, cm), stored(c[0], False, cm)
    lda, ldb, ldc = sa.shape[1] + case["pads"][0], sb.shape[1] + case["pads"][1], sc.shape[1] + case["pads"][2]
    A_e = [pad_rows(stored(x, ta, cm), lda, np.nan) for x in a]
    B_e = [pad_rows(stored(x, tb, cm), ldb, np.nan) for x in bm]
    C_e = [pad_rows(stored(x, False, cm), ldc, C_PAD_SENTINEL) for x in c]
    strides = [len(A_e[0]) + 3, len(B_e[0]) + 1, len(C_e[0]) + 2]
    A = np.full(strides[0] * batch, np.nan, np.float32)
    B = np.full(strides[1] * batch, np.nan, np.float32)
    C = np.full(strides[2] * batch, C_PAD_SENTINEL, np.float32)
    for i in range(batch):
        A[i * strides[0]: i * strides[0] + len(A_e[i])] = A_e[i]
        B[i * strides[1]: i * strides[1] + len(B_e[i])] = B_e[i]
        C[i * strides[2]: i * strides[2] + len(C_e[i])] = C_e[i]
    dA, dB, dC = device(A), device(B), device(C)
    fn = sgemm_cm_strided_batched_ws if cm else sgemm_rm_op_strided_batched_ws
    s = torch.cuda.current_stream()
    ws = ws_tensor.data_ptr() if case["ws"] else None
    fn(ta, tb, M, N, K, case["alpha"], dA.data_ptr(), lda, strides[0], dB.data_ptr(), ldb, strides[1],
       case["beta"], dC.data_ptr(), ldc, strides[2], batch, ws, WS_BYTES if case["ws"] else 0, s.cuda_stream,
       case["variant"])
    s.synchronize()
    out = dC.cpu().numpy()
    for i in range(batch):
        ref, _ = oracle.full(M, N, K, case["alpha"], a[i].reshape(-1), K, bm[i].reshape(-1), N, case["beta"],
                             c[i].reshape(-1), N)
        entry = out[i * strides[2]: i * strides[2] + len(C_e[i])]
        rows, cols = (N, M) if cm else (M, N)
        win = entry.reshape(rows, ldc)
        got = (win[:, :cols].T if cm else win[:, :cols]).astype(np.float64)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"case {case} entry {i}: {len(bad)} mismatches, first {bad[:3].tolist()}"
        pad_out = win[:, cols:].view(np.uint32)
        pad_in = C_e[i].reshape(rows, ldc)[:, cols:].view(np.uint32)
        assert np.array_equal(pad_out, pad_in), f"case {case} entry {i}: C padding written"
        gap = out[i * strides[2] + len(C_e[i]): (i + 1) * strides[2]]
        assert np.all(gap == np.float32(C_PAD_SENTINEL)), f"case {case}: gap after entry {i} written"


@pytest.mark.parametrize("block", range(6))
def test_random_sweep_integer_exact(oracle, block):
    """20 seeded random cases per block (120 in all)."""
    import torch

    ws_tensor = torch.empty(WS_BYTES, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(1000 + block)
    for t in range(20):
        case = draw_case(rng)
        run_case(oracle, case, seed=block * 100 + t, ws_tensor=ws_tensor)
