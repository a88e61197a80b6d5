"""The CRT-range failure flag on the GPU ([Q] section 時計の針で見る定理の中身:
outside (-P/2, P/2] the clocks read another number; [G] Problemstellung).

ozaki2_crt_check_debug reconstructs caller residues of chosen integers, in
range and wrapped, and flags each against one redundant modulus, compared
with the oracle's exact flags; ozaki2_dgemm_check runs real products with the
extra modulus and must flag nothing (the fast and accurate scalings keep the
range by construction) while writing the same C as ozaki2_dgemm_ws."""
import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import assert_bitwise_equal, device_colmajor, run_ws, stream_handle
import rns_emulated_fp64_amd as oz

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("N", [2, 8, 14, 16, 18, 19])
def test_check_flags_on_chosen_integers(N):
    moduli = O.choose_moduli(N)
    pc = O.check_modulus(N)
    P = math.prod(moduli)
    H = P // 2
    rng = np.random.default_rng(N)
    vals = [0, 1, -1, H, -H + 1, H - 1, H + 1, -H, -H - 1, P, -P, 2 * P + 3, -(pc - 1) * P, 3 * H]
    vals += [int(v) for v in rng.integers(-(1 << 62), 1 << 62, 30)]
    vals += [int(rng.integers(-(1 << 40), 1 << 40)) * (P >> 40) for _ in range(20)]  # large in range
    vals += [int(rng.integers(1, pc)) * P + int(rng.integers(-(1 << 30), 1 << 30)) for _ in range(20)]  # wrapped
    m, n = len(vals), 3
    Y = np.array([[v + j for j in range(n)] for v in vals], dtype=object)  # m x n
    c = np.stack([np.mod(Y, p) for p in moduli]).astype(np.int64)          # [N][m][n]
    cc = np.mod(Y, pc).astype(np.int64)
    want = O.crt_range_flags(c, cc, moduli, pc)                             # m x n
    X = O.crt(c, O.crt_tables(moduli))
    res = np.concatenate([c, cc[None]]).astype(np.uint8).transpose(0, 2, 1)  # [N+1][n][m]
    d_res = torch.from_numpy(np.ascontiguousarray(res)).cuda()
    e = torch.zeros(m, dtype=torch.int32, device="cuda")
    f = torch.zeros(n, dtype=torch.int32, device="cuda")
    C = torch.empty((n, m), dtype=torch.float64, device="cuda")
    flags = torch.full((n, m), 255, dtype=torch.uint8, device="cuda")
    wb = oz.ozaki2_check_workspace_size(m, n, 1, N, oz.FAST)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda")
    st = oz.ozaki2_crt_check_debug(m, n, N, d_res.data_ptr(), e.data_ptr(), f.data_ptr(), C.data_ptr(), m,
                                   flags.data_ptr(), ws.data_ptr(), wb, stream_handle())
    assert st == 0, oz.status_string(st)
    torch.cuda.synchronize()
    got = flags.cpu().numpy().T
    near = np.vectorize(lambda x: abs(2 * abs(int(x)) - P) * (1 << 30) < P)(X)  # |X| within 2^-30 P of P/2
    assert np.array_equal(got[~near], want[~near]), (got[~near], want[~near])
    assert np.all((got[near] == 2) | (got[near] == want[near]))
    # C is the reconstruction of the first N residues, rounded once
    assert_bitwise_equal(C.cpu().numpy().T, O.unscale(X, [0] * m, [0] * n), "C from the checked residues")


@pytest.mark.parametrize("m,n,k,N,mode", [(300, 200, 500, 8, "fast"), (257, 130, 1000, 14, "accurate"),
                                          (512, 512, 512, 16, "fast"), (100, 90, 777, 19, "fast")])
def test_dgemm_check_flags_nothing_on_scaled_products(m, n, k, N, mode):
    A, B = W.spread_case(m, n, k, 2.0, seed=m + n + k + N)
    md = oz.MODES[mode]
    dA, dB = device_colmajor(A), device_colmajor(B)
    C = torch.full((n, m), float("nan"), dtype=torch.float64, device="cuda")
    flags = torch.full((n, m), 255, dtype=torch.uint8, device="cuda")
    wb = oz.ozaki2_check_workspace_size(m, n, k, N, md)
    assert wb > oz.ozaki2_workspace_size(m, n, k, N, md)
    ws = torch.empty(wb, dtype=torch.uint8, device="cuda")
    st = oz.ozaki2_dgemm_check(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, C.data_ptr(), m, N, md, ws.data_ptr(),
                               wb, flags.data_ptr(), stream_handle())
    assert st == 0, oz.status_string(st)
    torch.cuda.synchronize()
    assert int(flags.max()) == 0
    assert_bitwise_equal(C.cpu().numpy().T, run_ws(A, B, N, mode), "check run vs _ws")
