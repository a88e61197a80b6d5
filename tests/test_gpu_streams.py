"""ozaki2_dgemm_ws is re-entrant: products on different streams, each with its
own workspace, may run at the same time. Four different products are
enqueued on four streams without synchronising between them, and each result
must equal, bit for bit, the same product computed alone."""
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


def test_concurrent_streams_match_sequential_products():
    cases = [(600, 520, 700, 16, "fast"), (300, 900, 450, 14, "accurate"), (1024, 256, 1024, 18, "fast"),
             (257, 263, 129, 8, "fast")]
    prepared = []
    for idx, (m, n, k, N, mode) in enumerate(cases):
        A, B = W.spread_case(m, n, k, 1.0, seed=70 + idx)
        md = oz.MODES[mode]
        wb = oz.ozaki2_workspace_size(m, n, k, N, md)
        prepared.append(dict(m=m, n=n, k=k, N=N, md=md, wb=wb, dA=device_colmajor(A), dB=device_colmajor(B),
                             ws=torch.empty(wb, dtype=torch.uint8, device="cuda"),
                             C=torch.full((n, m), float("nan"), dtype=torch.float64, device="cuda")))

    def enqueue(p, C, stream):
        st = oz.ozaki2_dgemm_ws(p["m"], p["n"], p["k"], p["dA"].data_ptr(), p["m"], p["dB"].data_ptr(), p["k"],
                                C.data_ptr(), p["m"], p["N"], p["md"], p["ws"].data_ptr(), p["wb"], stream)
        assert st == 0, oz.status_string(st)

    # alone, one after the other
    ref = []
    for p in prepared:
        C = torch.empty_like(p["C"])
        enqueue(p, C, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        ref.append(C.cpu().numpy())
    # all at once, each on its own stream, three rounds
    streams = [torch.cuda.Stream() for _ in prepared]
    for rnd in range(3):
        for p in prepared:
            p["C"].fill_(float("nan"))
        torch.cuda.synchronize()
        for p, s in zip(prepared, streams):
            enqueue(p, p["C"], s.cuda_stream)
        torch.cuda.synchronize()
        for i, p in enumerate(prepared):
            assert_bitwise_equal(p["C"].cpu().numpy(), ref[i], f"product {i}, round {rnd}")


def test_cached_workspace_calls_on_two_streams():
    # ozaki2_dgemm (no workspace argument) shares one cached workspace per
    # device; two different products enqueued back to back on two streams,
    # without synchronising in between, must each equal the oracle bit for bit
    # (the library orders their use of the workspace on the device)
    import oracle as O

    cases = [(1024, 1024, 1024, 14, "fast", 81), (768, 1024, 1024, 16, "accurate", 82)]
    prepared = []
    for m, n, k, N, mode, seed in cases:
        A, B = W.spread_case(m, n, k, 1.0, seed=seed)
        prepared.append(dict(m=m, n=n, k=k, N=N, md=oz.MODES[mode], dA=device_colmajor(A), dB=device_colmajor(B),
                             C=torch.empty((n, m), dtype=torch.float64, device="cuda"),
                             ref=O.os2_dgemm(A, B, N, mode)["C"]))
    streams = [torch.cuda.Stream() for _ in prepared]
    for rnd in range(3):
        for p in prepared:
            p["C"].fill_(float("nan"))
        torch.cuda.synchronize()
        for p, s in zip(prepared, streams):
            st = oz.ozaki2_dgemm(p["m"], p["n"], p["k"], p["dA"].data_ptr(), p["m"], p["dB"].data_ptr(), p["k"],
                                 p["C"].data_ptr(), p["m"], p["N"], p["md"], s.cuda_stream)
            assert st == 0, oz.status_string(st)
        torch.cuda.synchronize()
        for i, p in enumerate(prepared):
            assert_bitwise_equal(p["C"].cpu().numpy().T, p["ref"], f"cached product {i}, round {rnd}")
