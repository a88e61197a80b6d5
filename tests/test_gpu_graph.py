"""The caller-workspace entry points under HIP graph capture.

ozaki2_dgemm_ws / ozaki2_sgemm_ws / ozaki2_zgemm_ws enqueue kernels only (no allocation, no
memset, no host synchronisation), so a caller can capture a product into a
graph and replay it. Each test captures one call, then replays the graph
several times with new operands copied into the captured input buffers (eager
work and synchronisation between the replays) and checks every replay bit for
bit against an eager call on the same operands.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_bitwise_equal, device_colmajor
import rns_emulated_fp64_amd as oz

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oz.lib()


@pytest.mark.parametrize("kind,mode,N,shape", [
    ("d", "fast", 16, (300, 260, 700)),
    ("d", "accurate", 14, (300, 260, 700)),
    ("s", "fast", 8, (300, 260, 700)),
    # 4 x 5 tiles of 256 x 256 x 17 moduli = 340 > 256: the persistent GEMM in the graph
    ("d", "fast", 17, (1024, 1100, 520)),
    # complex: three planes per modulus, the reconstruction on the matrix cores
    ("z", "fast", 16, (300, 260, 700)),
])
def test_graph_replays_match_eager_calls(kind, mode, N, shape):
    m, n, k = shape
    single = kind == "s"
    cplx = kind == "z"
    call = oz.ozaki2_sgemm_ws if single else oz.ozaki2_zgemm_ws if cplx else oz.ozaki2_dgemm_ws
    dt = torch.float32 if single else torch.float64
    md = oz.MODES[mode]
    wb = oz.ozaki2_zgemm_workspace_size(m, n, k, N) if cplx else oz.ozaki2_workspace_size(m, n, k, N, md)
    ws_graph = torch.empty(wb, dtype=torch.uint8, device="cuda")
    ws_eager = torch.empty(wb, dtype=torch.uint8, device="cuda")

    def operands(seed):
        if cplx:
            from test_gpu_zgemm import complex_case, dev_complex
            A, B = complex_case(m, n, k, seed)
            return dev_complex(A, m, False), dev_complex(B, k, False)
        A, B = W.spread_case(m, n, k, 1.0, seed=seed)
        if single:
            A, B = A.astype(np.float32), B.astype(np.float32)
        return device_colmajor(A), device_colmajor(B)

    dA, dB = operands(40)
    dC = torch.full((n, m, 2) if cplx else (n, m), float("nan"), dtype=dt, device="cuda")

    def enqueue(A_, B_, C_, ws, stream):
        st = call(m, n, k, A_.data_ptr(), m, B_.data_ptr(), k, C_.data_ptr(), m, N, md, ws.data_ptr(), wb, stream)
        assert st == 0, oz.status_string(st)

    # warm-up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        enqueue(dA, dB, dC, ws_graph, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enqueue(dA, dB, dC, ws_graph, torch.cuda.current_stream().cuda_stream)

    for rep, seed in enumerate([41, 42, 43, 41]):
        nA, nB = operands(seed)
        dA.copy_(nA)
        dB.copy_(nB)
        dC.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = dC.cpu().numpy().copy()
        ref = torch.empty_like(dC)
        enqueue(nA, nB, ref, ws_eager, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert_bitwise_equal(got, ref.cpu().numpy(), f"replay {rep} ({kind}, {mode}, N={N})")
