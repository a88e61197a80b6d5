"""Timing hooks of the C ABI (ozaki2_timing_enable / ozaki2_timing_read) on
the GPU: the events ride on the phases' own kernel launches, change no bit of
C, give positive times for the timed phases and zero for the others, count
only the calls they have events for, and are cleared by a read."""
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


def teardown_function(function):
    oz.ozaki2_timing_enable(0)


@pytest.mark.parametrize("mode", ["fast", "accurate"])
def test_timing_changes_no_bit_and_reports_phases(mode):
    m, n, k, N = 300, 260, 1500, 16
    A, B = W.spread_case(m, n, k, 1.0, seed=11)
    dA, dB = device_colmajor(A), device_colmajor(B)
    md = oz.MODES[mode]
    wb = oz.ozaki2_workspace_size(m, n, k, N, md)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda")

    def run():
        dC = torch.empty((n, m), dtype=torch.float64, device="cuda")
        st = oz.ozaki2_dgemm_ws(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, dC.data_ptr(), m, N, md,
                                ws.data_ptr(), wb, stream_handle())
        assert st == 0, oz.status_string(st)
        return dC

    ref = run().cpu().numpy()
    outs = []

    # only the GEMM phase
    oz.ozaki2_timing_enable(3, all_phases=False)
    outs += [run(), run()]
    ms, calls = oz.ozaki2_timing_read()
    assert calls == 2
    assert ms["gemm"] > 0.0
    assert ms["scale"] == 0.0 and ms["split"] == 0.0 and ms["crt"] == 0.0

    # every phase; the kernels of one call run in order on one stream, so the
    # phase times are disjoint and each is far below a second at this size
    oz.ozaki2_timing_enable(2, all_phases=True)
    outs.append(run())
    ms, calls = oz.ozaki2_timing_read()
    assert calls == 1
    assert all(0.0 < v < 1000.0 for v in ms.values()), ms

    # a read clears the record
    ms, calls = oz.ozaki2_timing_read()
    assert calls == 0 and all(v == 0.0 for v in ms.values())

    # per call: one dict per timed call, summing to what the total read gives
    oz.ozaki2_timing_enable(3, all_phases=True)
    outs += [run(), run()]
    with pytest.raises(oz.Ozaki2Error):
        oz.ozaki2_timing_read_calls(1)  # too small: nothing cleared
    per = oz.ozaki2_timing_read_calls(3)
    assert len(per) == 2
    assert all(0.0 < c[p] < 1000.0 for c in per for p in oz.PHASES), per
    assert oz.ozaki2_timing_read_calls(3) == []

    # calls beyond the events created run untimed
    oz.ozaki2_timing_enable(1)
    outs += [run() for _ in range(3)]
    ms, calls = oz.ozaki2_timing_read()
    assert calls == 1 and ms["gemm"] > 0.0

    oz.ozaki2_timing_enable(0)
    outs.append(run())
    for i, o in enumerate(outs):
        assert_bitwise_equal(o.cpu().numpy(), ref, f"C of call {i}")


def test_timing_of_a_blocked_inner_dimension():
    # k beyond one GEMM launch (several accumulating launches): the GEMM phase
    # spans them all, from the first launch's start to the last one's end
    m, n, k, N = 40, 24, (1 << 16) + 64, 16
    A, B = W.uniform_case(m, n, k, seed=12)
    dA, dB = device_colmajor(A), device_colmajor(B)
    dC0 = torch.empty((n, m), dtype=torch.float64, device="cuda")
    dC1 = torch.empty((n, m), dtype=torch.float64, device="cuda")
    assert oz.ozaki2_dgemm(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, dC0.data_ptr(), m, N, 0, stream_handle()) == 0
    oz.ozaki2_timing_enable(1, all_phases=True)
    assert oz.ozaki2_dgemm(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, dC1.data_ptr(), m, N, 0, stream_handle()) == 0
    ms, calls = oz.ozaki2_timing_read()
    assert calls == 1 and all(v > 0.0 for v in ms.values()), ms
    assert_bitwise_equal(dC1.cpu().numpy(), dC0.cpu().numpy(), "C with timing on")
