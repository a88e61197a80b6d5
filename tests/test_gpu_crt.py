"""Steps 4 + 5 alone on the GPU (ozaki2_crt_debug) against the oracle, on
residue tuples chosen for their integers X rather than produced by a product.

Products of scaled operands keep |X| well inside (-P/2, P/2] and rarely come
near zero relative to P, so the exact wrap repair at +-P/2 and the branch for
a wrongly predicted sign of a tiny X are never reached through ozaki2_dgemm.
Here X is picked on those edges ([Q] section 時計の針で見る定理の中身: the
symmetric range (-P/2, P/2]), turned into residues c_l = X mod p_l, and the GPU
result must equal the oracle's RN(X) * 2^-(e_i + f_j) bit for bit, with NaN
rows and columns where the exponent marks a non-finite line.
"""
from __future__ import annotations

import random

import numpy as np
import pytest
import torch

import oracle as O
import rns_emulated_fp64_amd as oz
from gpu_util import INT32_MIN, assert_bitwise_equal, stream_handle

pytestmark = pytest.mark.gpu


def edge_values(P: int) -> list[int]:
    """Integers in (-P/2, P/2] on every edge the reconstruction treats apart."""
    H = P // 2  # P is even (256 is always a modulus)
    vals = {0, 1, -1, 2, -2, H, H - 1, H - 2, -H + 1, -H + 2, -H + 3}
    # the quotient estimate's decision band: |X/P| within 2^-30 of 1/2
    for sh in (24, 30, 31, 36):
        d = P >> sh
        vals.update({H - d, H - d - 1, H - d + 1, -H + d, -H + d + 1, -H + d - 1})
    # tiny X, where the sign read from the estimate is unreliable
    for sh in (30, 37, 38, 45, 60, 90):
        d = P >> sh
        vals.update({d, -d, d + 1, -d - 1})
    # powers of two and their neighbours over the whole range
    b = 0
    while (1 << b) <= H:
        vals.update({1 << b, -(1 << b), (1 << b) - 1, -(1 << b) + 1, (1 << b) + 1})
        b += 1
    return sorted(v for v in vals if -H < v <= H)


def crafted_case(N: int, seed: int):
    moduli = O.choose_moduli(N)
    P = O.crt_tables(moduli)["P"]
    rnd = random.Random(seed)
    vals = edge_values(P)
    H = P // 2
    vals += [rnd.randrange(-H + 1, H + 1) for _ in range(300)]
    n = 7
    m = (len(vals) + n - 1) // n
    vals += [rnd.randrange(-H + 1, H + 1) for _ in range(m * n - len(vals))]
    rnd.shuffle(vals)
    X = np.empty((m, n), dtype=object)
    for idx, v in enumerate(vals):
        X[idx % m, idx // m] = v
    e = [rnd.randrange(-40, 41) for _ in range(m)]
    f = [rnd.randrange(-40, 41) for _ in range(n)]
    e[3] = None          # a row that held Inf/NaN
    f[5] = None
    bits = (P // 2).bit_length()
    e[4] = bits + 1040   # results in the subnormal range ...
    e[6] = bits + 1075   # ... and below it
    e[7] = -800          # large results
    return moduli, P, X, e, f


@pytest.mark.parametrize("N", [2, 3, 8, 14, 15, 16, 17, 18, 19, 20])
def test_crt_edges_bitwise(N):
    _crt_edges(N)


@pytest.mark.parametrize("N", [17, 18, 19, 20])
def test_crt_edges_bitwise_fma_form(monkeypatch, N):
    # 17..20 moduli run on the matrix cores by default; OZ2_CRT=fma keeps the
    # FP64-FMA form on 40-bit pieces, which must agree on the same edges
    monkeypatch.setenv("OZ2_CRT", "fma")
    _crt_edges(N)


def _crt_edges(N):
    moduli, P, X, e, f = crafted_case(N, 1000 + N)
    m, n = X.shape
    c = np.empty((N, n, m), dtype=np.uint8)  # [l][j][i], values in [0, p_l)
    for l, p in enumerate(moduli):
        c[l] = np.vectorize(lambda v: v % p, otypes=[object])(X).T.astype(np.uint8)
    # the residues name exactly these integers
    back = O.crt(np.transpose(c, (0, 2, 1)).astype(np.int64), O.crt_tables(moduli))
    assert all(int(back[i, j]) == X[i, j] for i in range(m) for j in range(n))
    expect = O.unscale(X, e, f)

    dres = torch.from_numpy(c).cuda()
    de = torch.tensor([INT32_MIN if v is None else v for v in e], dtype=torch.int32, device="cuda")
    df = torch.tensor([INT32_MIN if v is None else v for v in f], dtype=torch.int32, device="cuda")
    ldc = m + 3
    dC = torch.full((n, ldc), 7.0, dtype=torch.float64, device="cuda")
    wbytes = oz.ozaki2_workspace_size(m, n, 1, N, oz.FAST)
    ws = torch.empty(wbytes, dtype=torch.uint8, device="cuda")
    st = oz.ozaki2_crt_debug(m, n, N, dres.data_ptr(), de.data_ptr(), df.data_ptr(), dC.data_ptr(), ldc,
                             ws.data_ptr(), wbytes, stream_handle())
    assert st == 0, oz.status_string(st)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    assert_bitwise_equal(out[:, :m].T.copy(), expect, f"CRT N={N}")
    assert np.all(out[:, m:] == 7.0), "wrote outside the m rows of C"
    # the edge set really reaches the subnormal range and both wrap ends
    assert np.any((expect != 0) & (np.abs(expect) < np.finfo(np.float64).tiny))
    assert X.max() == P // 2 and X.min() == -(P // 2) + 1

