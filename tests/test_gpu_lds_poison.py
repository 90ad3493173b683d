"""Reads of unwritten LDS: every kernel family and tile form on the LDS-poisoning build.

`libsgemm_rm_poison.so` is the library compiled with SGEMM_RM_POISON_LDS: each kernel
that uses LDS fills all of it with NaN before anything else.  A read of LDS that no thread
of the launch has written (a missing barrier, a part of a tile left unfilled, a stage read
before its store) then reaches C as NaN, even where its value is multiplied by zero.  The
m.lqnn.cn/news/94381 page warns in section 3.2 (and step 3 of section 6.1) that a missing
barrier or unfilled shared memory gives results that are right only sometimes; poisoning
makes such a read fail every time.

Integer inputs in [-4, 4] with NaN padding in A and B make every result exact, so each
case is compared bit for bit with the oracle, over every output, and C's padding must be
untouched.  The cases reach each LDS layout and pipeline: the LDS-tiled and
register-blocked VALU kernels, every forced MFMA tile configuration with full, guarded and
thin-strip partial tiles, the fused right strip, the 256 configuration's thin-strip form,
scalar edge tiles and LDS-DMA loads, stream-K pieces with their fix-up, K slices with theirs,
16 x 16 blocks, the one-layer 128 form, a strided batch, transposed operands and K tails.
"""
import numpy as np
import pytest

from fp32_gemm_rm_amd.workloads import C_PAD_SENTINEL, integer_matrix, pad_rows

from .parity import c_window, check_padding, device

pytestmark = pytest.mark.gpu

# (variant, transA, transB, M, N, K, batch, stream-K workspace)
CASES = [
    (2, 0, 0, 300, 270, 145, 1, False), (2, 1, 1, 33, 65, 17, 1, False),  # LDS-tiled
    (3, 0, 0, 300, 270, 145, 1, False), (3, 1, 0, 129, 200, 99, 1, False),  # register-blocked
    (5, 0, 0, 2 * 256 + 4, 256 + 3, 70, 1, False),  # 256: thin strips after the tiles
    (5, 0, 1, 256 + 40, 256 + 33, 45, 1, False),  # 256: scalar edge tiles
    (9, 0, 0, 2 * 192 + 32, 192 + 31, 70, 1, False), (9, 1, 0, 192 + 15, 2 * 192 + 16, 45, 1, False),
    (6, 0, 0, 3 * 128 + 32, 2 * 128 + 31, 70, 1, False), (6, 0, 1, 2 * 128 + 7, 3 * 128 + 1, 70, 1, False),
    (6, 0, 0, 256, 384, 16 * 9 + 5, 1, False),  # 128: the one-layer form
    (7, 0, 0, 5 * 64 + 16, 4 * 64 + 15, 70, 1, False), (7, 1, 1, 64 + 15, 64 + 15, 70, 1, False),
    (7, 0, 0, 1000, 1030, 999, 1, False),  # 64: right strip inside the tiles
    (7, 0, 0, 3 * 64 + 5, 16 * 64 + 3, 700, 1, False),
    (8, 0, 0, 3 * 32 + 2, 2 * 32 + 3, 70, 1, False), (8, 1, 0, 2 * 32 + 6, 3 * 32 + 6, 300, 1, False),
    (10, 0, 0, 17, 33, 70, 1, False), (10, 0, 1, 5 * 16 + 3, 3 * 16 + 9, 1100, 1, False),
    (0, 0, 0, 70, 50, 33, 7, False),  # strided batch, default path
    # 256 tiles through LDS-DMA loads (16-byte rows, K a multiple of 16): fewer K-tiles than
    # stages and transposed, thin strips beside them, a strided batch
    (5, 0, 0, 512, 768, 144, 1, False), (5, 1, 1, 512, 512, 48, 1, False), (5, 0, 1, 256 + 8, 512, 160, 1, False),
    (5, 0, 0, 256, 256, 64, 3, False),
    (5, 0, 0, 256 + 40, 512 + 24, 144, 1, False), (5, 1, 0, 300, 520, 64, 1, False),  # guarded direct tiles
    (5, 0, 1, 256 + 16, 256 + 18, 48, 1, False),  # guarded direct tiles and a 2-column thin strip
    # the 128 configuration's two-workgroup form (more than 256 tiles) through LDS-DMA loads
    (6, 0, 0, 2100, 2090, 160, 1, False), (6, 0, 1, 2060, 2100, 48, 1, False),
    (6, 1, 1, 2060, 2100, 48, 1, False), (7, 1, 0, 1130, 1110, 64, 1, False),  # A^T
    # the 192 configuration and the 128 one-layer form on LDS-DMA loads
    (9, 0, 0, 3 * 192 + 40, 2 * 192 + 20, 96, 1, False), (9, 1, 0, 420, 400, 64, 1, False),
    (6, 1, 1, 300, 296, 64, 1, False),
    # and the 64 one's (K a multiple of 32), with two workgroups per CU or one
    (7, 0, 0, 1000, 1000, 96, 1, False), (7, 0, 1, 1060, 1000, 40, 1, False),  # the last with a partial K-tile
    (7, 0, 0, 1130, 1110, 64, 1, False), (7, 0, 1, 1100, 1090, 96, 1, False),
    (5, 0, 0, 1024, 1280, 77, 1, True),  # stream-K (256 forced, with a workspace): every tile split
    (5, 0, 0, 17 * 256, 17 * 256, 40, 1, True),  # stream-K: whole tiles and pieces
    (7, 0, 0, 210, 148, 30000, 1, True),  # K slices (64 forced, with a workspace) and their fix-up
]


def _stored(x, trans, ld, pad):
    """Logical rows x cols matrix x stored row-major (trans: its transpose), leading
    dimension ld, padding `pad`."""
    y = np.ascontiguousarray(x.T) if trans else x
    return pad_rows(y, ld, pad)


@pytest.fixture(scope="module")
def lib():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp32_gemm_rm_amd.binding import load_library, load_poison_library

    load_library()
    return load_poison_library()


@pytest.mark.parametrize("variant,ta,tb,M,N,K,batch,use_ws", CASES)
def test_poisoned_lds_integer_exact(oracle, lib, variant, ta, tb, M, N, K, batch, use_ws):
    import torch

    print(f"[poison] variant={variant} op={ta}{tb} {M}x{N}x{K} batch={batch} ws={use_ws}", flush=True)
    lda, ldb, ldc = (M if ta else K) + 4, (K if tb else N) + 4, N + 1
    rows_a, rows_b = (K if ta else M), (N if tb else K)
    sA, sB, sC = rows_a * lda, rows_b * ldb, M * ldc
    As, Bs, Cs, refs = [], [], [], []
    for e in range(batch):
        a = integer_matrix(M, K, -4, 4, seed=M + 3 * K + e)
        b = integer_matrix(K, N, -4, 4, seed=N + 3 * K + e)
        c = integer_matrix(M, N, -4, 4, seed=M + 3 * N + e)
        As.append(_stored(a, ta, lda, np.nan))
        Bs.append(_stored(b, tb, ldb, np.nan))
        Cs.append(pad_rows(c, ldc, C_PAD_SENTINEL))
        ref, _ = oracle.full(M, N, K, -1.5, a.reshape(-1), K, b.reshape(-1), N, 0.5, Cs[-1], ldc, with_absab=False)
        refs.append(ref)
    dA, dB, dC = device(np.concatenate(As)), device(np.concatenate(Bs)), device(np.concatenate(Cs))
    from fp32_gemm_rm_amd.binding import SGEMM_RM_SCRATCH_BYTES

    need = SGEMM_RM_SCRATCH_BYTES if use_ws else 0  # the stream-K / K-slice workspace (128 MiB)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    rc = lib.sgemm_rm_op_strided_batched_ws(ta, tb, M, N, K, -1.5, dA.data_ptr(), lda, sA, dB.data_ptr(), ldb, sB,
                                            0.5, dC.data_ptr(), ldc, sC, batch, ws.data_ptr() if need else None,
                                            need, s.cuda_stream, variant)
    assert rc == 0, rc
    s.synchronize()
    out = dC.cpu().numpy()
    for e in range(batch):
        got = c_window(out[e * sC:(e + 1) * sC], M, N, ldc).astype(np.float64)
        assert not np.isnan(got).any(), f"entry {e}: NaN in C, a read of unwritten LDS"
        bad = np.argwhere(got != refs[e])
        assert bad.size == 0, f"entry {e}: {len(bad)} mismatches, first at {bad[:3].tolist()}"
        check_padding(out[e * sC:(e + 1) * sC], Cs[e], M, N, ldc)
