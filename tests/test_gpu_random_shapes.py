"""Seeded random sweep of shapes, moduli counts, modes and leading
dimensions, each checked stage by stage against the oracle (exponents under
the boundary protocol; int8 residues, int32 products, reduced residues and C
bit-exact). The sizes cluster next to the kernels' boundaries: 1..40 and
250..262 rows or columns (one 256-wide tile and a ragged second one), inner
dimensions next to multiples of 64 and 128 (stage and split-tile widths).

Pages: [Q] steps 1-5; [G] section Methodik.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import full_parity
import rns_emulated_fp64_amd as oz

pytestmark = pytest.mark.gpu


def _cases(seed=2026, count=48):
    rng = np.random.default_rng(seed)
    pick = lambda ranges: int(rng.integers(*ranges[int(rng.integers(len(ranges)))]))
    out = []
    for _ in range(count):
        m = pick([(1, 41), (250, 263)])
        n = pick([(1, 41), (250, 263)])
        k = pick([(1, 70), (120, 136), (250, 262), (1000, 1031)])
        N = int(rng.integers(2, 21))
        mode = "accurate" if rng.random() < 0.3 else "fast"
        phi = float(rng.choice([0.5, 1.0, 2.0]))
        pads = [int(x) for x in rng.integers(0, 4, size=3)]
        out.append((m, n, k, N, mode, phi, pads, int(rng.integers(1 << 30))))
    return out


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oz.lib()


@pytest.mark.parametrize("m,n,k,N,mode,phi,pads,seed", _cases(),
                         ids=lambda v: None if not isinstance(v, tuple) else str(v))
def test_random_shape(m, n, k, N, mode, phi, pads, seed):
    A, B = W.spread_case(m, n, k, phi, seed=seed)
    full_parity(A, B, N, mode, lda=m + pads[0], ldb=k + pads[1], ldc=m + pads[2], want_prod=True)


def _complex_cases(seed=2027, count=16):
    rng = np.random.default_rng(seed)
    pick = lambda ranges: int(rng.integers(*ranges[int(rng.integers(len(ranges)))]))
    out = []
    for _ in range(count):
        m = pick([(1, 41), (250, 263)])
        n = pick([(1, 41), (250, 263)])
        k = pick([(1, 70), (120, 136), (250, 262)])
        N = int(rng.integers(2, 21))
        single = bool(rng.random() < 0.4)
        pads = [int(x) for x in rng.integers(0, 4, size=3)]
        out.append((m, n, k, N, single, pads, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("m,n,k,N,single,pads,seed", _complex_cases(),
                         ids=lambda v: None if not isinstance(v, tuple) else str(v))
def test_random_shape_complex(m, n, k, N, single, pads, seed):
    # complex products (ZGEMM, or CGEMM on binary32 operands): three residue
    # planes per modulus, every stage bit-exact against the oracle
    from test_gpu_zgemm import complex_case, complex_parity
    A, B = complex_case(m, n, k, seed)
    if single:
        A, B = A.astype(np.complex64), B.astype(np.complex64)
    complex_parity(A, B, N, single, lda=m + pads[0], ldb=k + pads[1], ldc=m + pads[2])


@pytest.mark.parametrize("m,n,k,N,mode,phi,pads,seed", _cases(seed=2028, count=16),
                         ids=lambda v: None if not isinstance(v, tuple) else str(v))
def test_random_shape_single(m, n, k, N, mode, phi, pads, seed):
    # binary32 operands through ozaki2_sgemm_debug: every stage bit-exact,
    # C rounded once to binary32 as the oracle's os2_sgemm does
    A, B = W.spread_case(m, n, k, phi, seed=seed)
    full_parity(A.astype(np.float32), B.astype(np.float32), N, mode, lda=m + pads[0], ldb=k + pads[1],
                ldc=m + pads[2], want_prod=True)


@pytest.mark.parametrize("tile", ["128", "256"])
@pytest.mark.parametrize("m,n,k,N,mode,phi,pads,seed", _cases(seed=2029, count=8),
                         ids=lambda v: None if not isinstance(v, tuple) else str(v))
def test_random_shape_each_tile_shape(monkeypatch, tile, m, n, k, N, mode, phi, pads, seed):
    # the GEMM has a 256 x 256 and a 128 x 128 block shape, chosen by problem
    # size; forcing each one here runs both on every shape
    monkeypatch.setenv("OZ2_GEMM_TILE", tile)
    A, B = W.spread_case(m, n, k, phi, seed=seed)
    full_parity(A, B, N, mode, lda=m + pads[0], ldb=k + pads[1], ldc=m + pads[2], want_prod=True)
