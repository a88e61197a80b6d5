"""The complex reconstruction alone (ozaki2_zcrt_debug) against the oracle, on
residue triples chosen for the integers they name.

Per modulus the three products give residues T1, T2, T3, and the parts are
Re = T1 - T2, Im = T3 - T1 - T2 (Gauss' three-multiplication form, exact in
residues). Targets Xr, Xi are picked on the edges of (-P/2, P/2] ([Q] section
時計の針で見る定理の中身) and at random; T1 is drawn (uniformly, or at the ends
of the symmetric range so that T1 - T2 and T3 - T1 - T2 reach their largest
magnitudes), then T2 = T1 - Xr and T3 = Xi + T1 + T2 mod p. Both parts of C
must equal the oracle's RN(X) * 2^-(e_i + f_j) bit for bit, on the matrix-core
forms (the default for 2..20 moduli) and on the FP64-FMA form (OZ2_CRT=fma).
"""
from __future__ import annotations

import random

import numpy as np
import pytest
import torch

import oracle as O
import rns_emulated_fp64_amd as oz
from gpu_util import INT32_MIN, assert_bitwise_equal, stream_handle
from test_gpu_crt import edge_values

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def crafted_case(N: int, seed: int, extreme: bool):
    moduli = O.choose_moduli(N)
    P = O.crt_tables(moduli)["P"]
    H = P // 2
    rnd = random.Random(seed)
    vals = edge_values(P) + [rnd.randrange(-H + 1, H + 1) for _ in range(200)]
    n = 7
    m = (len(vals) + n - 1) // n
    vals += [rnd.randrange(-H + 1, H + 1) for _ in range(m * n - len(vals))]
    Xr = np.empty((m, n), dtype=object)
    Xi = np.empty((m, n), dtype=object)
    a, b = list(vals), list(vals)
    rnd.shuffle(a)
    rnd.shuffle(b)
    for idx in range(m * n):
        Xr[idx % m, idx // m] = a[idx]
        Xi[idx % m, idx // m] = b[idx]
    T = np.empty((3 * N, n, m), dtype=np.uint8)  # [3l + g][j][i], values in [0, p_l)
    for l, p in enumerate(moduli):
        lo, hi = (p - 1) // 2 + 1, (p - 1) // 2  # most negative / most positive symmetric residue
        for i in range(m):
            for j in range(n):
                t1 = rnd.choice((lo, hi)) if extreme else rnd.randrange(p)
                t2 = (t1 - Xr[i, j]) % p
                t3 = (Xi[i, j] + t1 + t2) % p
                T[3 * l, j, i], T[3 * l + 1, j, i], T[3 * l + 2, j, i] = t1, t2, t3
    e = [rnd.randrange(-40, 41) for _ in range(m)]
    f = [rnd.randrange(-40, 41) for _ in range(n)]
    e[3] = None  # a row that held Inf/NaN
    f[5] = None
    bits = H.bit_length()
    e[4] = bits + 1040  # subnormal results ...
    e[6] = bits + 1075  # ... and below
    e[7] = -800
    return moduli, P, T, Xr, Xi, e, f


def _zcrt(N: int, extreme: bool):
    moduli, P, T, Xr, Xi, e, f = crafted_case(N, 2000 + N + (7 if extreme else 0), extreme)
    _, n, m = T.shape
    # the residues name exactly these parts (oracle's own reduction and CRT)
    t = T.astype(np.int64).reshape(N, 3, n, m).transpose(0, 1, 3, 2)  # [l][g][i][j]
    tables = O.crt_tables(moduli)
    back_r = O.crt(O.reduce_products(t[:, 0] - t[:, 1], moduli), tables)
    back_i = O.crt(O.reduce_products(t[:, 2] - t[:, 0] - t[:, 1], moduli), tables)
    assert all(int(back_r[i, j]) == Xr[i, j] and int(back_i[i, j]) == Xi[i, j] for i in range(m) for j in range(n))
    exp_r, exp_i = O.unscale(Xr, e, f), O.unscale(Xi, e, f)

    dres = torch.from_numpy(T).cuda()
    de = torch.tensor([INT32_MIN if v is None else v for v in e], dtype=torch.int32, device="cuda")
    df = torch.tensor([INT32_MIN if v is None else v for v in f], dtype=torch.int32, device="cuda")
    ldc = m + 3
    dC = torch.full((n, ldc, 2), 7.0, dtype=torch.float64, device="cuda")
    wbytes = oz.ozaki2_zgemm_workspace_size(m, n, 1, N)
    ws = torch.empty(wbytes, dtype=torch.uint8, device="cuda")
    st = oz.ozaki2_zcrt_debug(m, n, N, dres.data_ptr(), de.data_ptr(), df.data_ptr(), dC.data_ptr(), ldc,
                              ws.data_ptr(), wbytes, stream_handle())
    assert st == 0, oz.status_string(st)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    assert_bitwise_equal(out[:, :m, 0].T.copy(), exp_r, f"Re, N={N}")
    assert_bitwise_equal(out[:, :m, 1].T.copy(), exp_i, f"Im, N={N}")
    assert np.all(out[:, m:, :] == 7.0), "wrote outside the m rows of C"
    assert max(Xr.max(), Xi.max()) == P // 2 and min(Xr.min(), Xi.min()) == -(P // 2) + 1


# 2..7 moduli: two 32-bit pieces, 8..12: three, 13..16: four; 17..20: five
# (two digit blocks per part); all on the matrix cores by default
@pytest.mark.parametrize("N", [2, 5, 8, 12, 13, 16, 17, 18, 19, 20])
@pytest.mark.parametrize("extreme", [False, True])
def test_zcrt_edges_bitwise(N, extreme):
    _zcrt(N, extreme)


@pytest.mark.parametrize("N", [3, 9, 16, 18, 20])
def test_zcrt_edges_bitwise_fma_form(monkeypatch, N):
    monkeypatch.setenv("OZ2_CRT", "fma")
    _zcrt(N, True)


def test_zcrt_argument_errors():
    assert oz.ozaki2_zcrt_debug(-1, 1, 4, 0, 0, 0, 0, 1, 0, 0) == -1
    assert oz.ozaki2_zcrt_debug(1, 1, 1, 0, 0, 0, 0, 1, 0, 0) == -3
    assert oz.ozaki2_zcrt_debug(0, 3, 4, 0, 0, 0, 0, 1, 0, 0) == 0  # empty: nothing to do
    assert oz.ozaki2_zcrt_debug(4, 1, 4, 0, 0, 0, 0, 4, 0, 0) == -4
