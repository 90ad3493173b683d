"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph).

Every entry point only enqueues kernels on the caller's stream and calls no allocator,
memset or synchronisation, so a capture records its kernels and replays repeat them.
Each replay is compared with the eager result of the same call (bitwise: same kernels,
same order), with eager work and host synchronisation between replays.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

WS_BYTES = 2 * 256 * 256 * 256 * 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp32_gemm_rm_amd import load_library

    load_library()


def test_graph_replays_match_eager(oracle):
    import torch

    from fp32_gemm_rm_amd import sgemm_rm_ex, sgemm_rm_op_strided_batched_ws, sgemm_rm_strided_batched_ex

    gen = torch.Generator(device="cuda").manual_seed(3)
    # four calls on four paths: 32x32 tiles with guarded partial tiles, a strided batch,
    # stream-K (forced 256 tiles with a workspace: 20 tiles, a partial wave) and K slices
    # (the default path with a workspace: 4 tiles of 64 x 64, each K range in 64 slices)
    A1, B1 = torch.randn(300, 257, device="cuda", generator=gen), torch.randn(257, 190, device="cuda", generator=gen)
    A2, B2 = torch.randn(8, 64, 96, device="cuda", generator=gen), torch.randn(8, 96, 80, device="cuda", generator=gen)
    A3, B3 = torch.randn(1024, 200, device="cuda", generator=gen), torch.randn(200, 1280, device="cuda", generator=gen)
    C1, C2 = torch.empty(300, 190, device="cuda"), torch.empty(8, 64, 80, device="cuda")
    C3 = torch.empty(1024, 1280, device="cuda")
    A4, B4 = torch.randn(128, 40000, device="cuda", generator=gen), torch.randn(40000, 128, device="cuda", generator=gen)
    C4 = torch.empty(128, 128, device="cuda")
    ws = torch.empty(WS_BYTES, dtype=torch.uint8, device="cuda")
    ws4 = torch.empty(WS_BYTES, dtype=torch.uint8, device="cuda")

    def calls(stream):
        s = stream.cuda_stream
        sgemm_rm_ex(300, 190, 257, 1.0, A1.data_ptr(), 257, B1.data_ptr(), 190, 0.0, C1.data_ptr(), 190, s, 0)
        sgemm_rm_strided_batched_ex(64, 80, 96, 0.5, A2.data_ptr(), 96, 64 * 96, B2.data_ptr(), 80, 96 * 80, 0.0,
                                    C2.data_ptr(), 80, 64 * 80, 8, s, 0)
        sgemm_rm_op_strided_batched_ws(0, 0, 1024, 1280, 200, 1.0, A3.data_ptr(), 200, 0, B3.data_ptr(), 1280, 0,
                                       0.0, C3.data_ptr(), 1280, 0, 1, ws.data_ptr(), WS_BYTES, s, 5)
        sgemm_rm_op_strided_batched_ws(0, 0, 128, 128, 40000, 1.0, A4.data_ptr(), 40000, 0, B4.data_ptr(), 128, 0,
                                       0.0, C4.data_ptr(), 128, 0, 1, ws4.data_ptr(), WS_BYTES, s, 0)

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        calls(side)
    side.synchronize()
    eager = [C1.clone(), C2.clone(), C3.clone(), C4.clone()]

    graph = torch.cuda.CUDAGraph()
    for C in (C1, C2, C3, C4):
        C.fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        calls(torch.cuda.current_stream())
    for rep in range(4):
        for C in (C1, C2, C3, C4):
            C.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (C, E) in enumerate(zip((C1, C2, C3, C4), eager)):
            assert torch.equal(C, E), f"replay {rep}, call {k}"
    # and the eager results are right
    a, b = A3.cpu().numpy().reshape(-1), B3.cpu().numpy().reshape(-1)
    ref, S = oracle.full(1024, 1280, 200, 1.0, a, 200, b, 1280, 0.0, None, 1280)
    assert np.all(np.abs(eager[2].cpu().numpy().astype(np.float64) - ref) <= 1e-5 * S + 1e-6)
    a, b = A4.cpu().numpy().reshape(-1), B4.cpu().numpy().reshape(-1)
    ref, S = oracle.full(128, 128, 40000, 1.0, a, 40000, b, 128, 0.0, None, 128)
    assert np.all(np.abs(eager[3].cpu().numpy().astype(np.float64) - ref) <= 1e-5 * S + 1e-6)
