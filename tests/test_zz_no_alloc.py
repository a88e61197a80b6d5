"""ozaki2_dgemm_noalloc: the product with its workspace in the library's
static device array (for callers that cannot allocate device memory) must
equal ozaki2_dgemm_ws bit for bit, call after call: two products in a row on
one GPU, the second smaller than the first, so the second runs on an array
still holding the first one's contents."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_bitwise_equal, device_colmajor, stream_handle
import rns_emulated_fp64_amd as oz

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oz.lib()


def _ws_product(dA, dB, m, n, k, N, md):
    C = torch.full((n, m), float("nan"), dtype=torch.float64, device="cuda")
    wb = oz.ozaki2_workspace_size(m, n, k, N, md)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda")
    st = oz.ozaki2_dgemm_ws(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, C.data_ptr(), m, N, md, ws.data_ptr(), wb,
                            stream_handle())
    assert st == 0, oz.status_string(st)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def test_noalloc_equals_ws_on_two_calls_in_a_row():
    cases = [(1000, 900, 1100, 16, "fast", 91), (300, 200, 257, 14, "accurate", 92)]
    for m, n, k, N, mode, seed in cases:
        md = oz.MODES[mode]
        assert oz.ozaki2_workspace_size(m, n, k, N, md) <= oz.NOALLOC_MAX_WORKSPACE
        A, B = W.spread_case(m, n, k, 1.0, seed=seed)
        dA, dB = device_colmajor(A), device_colmajor(B)
        ref = _ws_product(dA, dB, m, n, k, N, md)
        C = torch.full((n, m), float("nan"), dtype=torch.float64, device="cuda")
        print(f"noalloc {m}x{n}x{k} N={N} {mode}", flush=True)
        st = oz.ozaki2_dgemm_noalloc(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, C.data_ptr(), m, N, md,
                                     stream_handle())
        assert st == 0, oz.status_string(st)
        torch.cuda.synchronize()
        assert_bitwise_equal(C.cpu().numpy(), ref, f"noalloc {m}x{n}x{k} N={N} {mode}")


def test_noalloc_refuses_products_beyond_its_array():
    # 2048^3 at 16 moduli needs about 200 MiB of workspace: refused before any
    # device work, C untouched
    m = n = k = 2048
    assert oz.ozaki2_workspace_size(m, n, k, 16, 0) > oz.NOALLOC_MAX_WORKSPACE
    C = torch.zeros((n, m), dtype=torch.float64, device="cuda")
    A = torch.ones((k, m), dtype=torch.float64, device="cuda")
    st = oz.ozaki2_dgemm_noalloc(m, n, k, A.data_ptr(), m, A.data_ptr(), k, C.data_ptr(), m, 16, 0, stream_handle())
    assert st == oz.ERR_NOALLOC_LIMIT
    torch.cuda.synchronize()
    assert float(C.abs().max()) == 0.0
