"""The persistent form of the 256 x 256 INT8 GEMM (one block per compute unit
walking its tiles, the copy ring running across tile boundaries; the default
when there are more tiles than compute units and a launch has at least four
64-deep stages; OZ2_GEMM_KERNEL=persistent forces it) against the
one-tile-per-block kernel (OZ2_GEMM_KERNEL=blocks) and against the oracle: the reduced residue
planes and C bit-identical. Shapes cover one tile per block, a grid of more
tiles than compute units (blocks walking two tiles, a ragged last round), the
shortest inner dimension it takes (four stages), an inner dimension split into
accumulating launches whose second one still has four or more stages, and
complex products (three planes per modulus).

Pages: [Q] step 3 (one exact INT8 product per modulus, reduced mod p)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from gpu_util import assert_bitwise_equal, full_parity, run_debug

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both_kernels(monkeypatch, A, B, N, mode="fast"):
    monkeypatch.setenv("OZ2_GEMM_TILE", "256")
    monkeypatch.setenv("OZ2_GEMM_KERNEL", "blocks")
    g0 = run_debug(A, B, N, mode, want_prod=False, want_res=False)
    monkeypatch.setenv("OZ2_GEMM_KERNEL", "persistent")
    g1 = run_debug(A, B, N, mode, want_prod=False, want_res=False)
    assert np.array_equal(g1["red"], g0["red"]), "reduced residue planes differ between the two kernels"
    assert_bitwise_equal(g1["C"], g0["C"], "C (persistent vs blocks)")
    return g1


# (m, n, k, N): tiles = ceil(m/256) * ceil(n/256) * N
SHAPES = [
    (256, 256, 256, 2),      # one tile per block, exactly four stages
    (300, 200, 200, 8),      # ragged edges, k padded to 256
    (700, 530, 390, 20),     # 3 x 3 x 20 = 180 tiles
    (1100, 1100, 300, 11),   # 5 x 5 x 11 = 275 tiles: 19 blocks walk a second tile
    (1024, 1024, 1000, 20),  # 320 tiles, 16 stages
    (1500, 1500, 256, 16),   # 6 x 6 x 16 = 576 tiles: two or three per block, four stages each
]


@pytest.mark.parametrize("m,n,k,N", SHAPES)
def test_persistent_equals_blocks_kernel(monkeypatch, m, n, k, N):
    A, B = W.spread_case(m, n, k, 1.0, seed=m + n + k + N)
    _both_kernels(monkeypatch, A, B, N)


def test_persistent_accurate_mode(monkeypatch):
    A, B = W.spread_case(600, 900, 700, 2.0, seed=41)
    _both_kernels(monkeypatch, A, B, 16, "accurate")


def test_persistent_walking_tiles_against_oracle():
    # 4 x 4 tiles x 17 moduli = 272 > 256 blocks (the persistent kernel by
    # default), so some blocks take a second tile and its first stages are
    # copied during the first tile's epilogue
    A, B = W.spread_case(1024, 1024, 300, 1.0, seed=17)
    full_parity(A, B, 17, want_prod=False)


def test_persistent_forced_against_oracle(monkeypatch):
    # fewer tiles than compute units: the block kernel by default, the
    # persistent one when forced (one tile per block)
    monkeypatch.setenv("OZ2_GEMM_KERNEL", "persistent")
    A, B = W.spread_case(700, 530, 390, 1.0, seed=18)
    full_parity(A, B, 12, want_prod=False)


@pytest.mark.parametrize("k", [65536 + 300, 65536 + 200])
def test_persistent_split_inner_dimension(monkeypatch, k):
    # k_pad = 65536 + 384 (65536 + 256): launches of 1024 and 6 (4) stages;
    # the second one adds to the residues of the first (the accumulating
    # epilogue) and is still long enough for the persistent kernel
    A, B = W.spread_case(260, 40, k, 0.5, seed=3)
    g = _both_kernels(monkeypatch, A, B, 8)
    assert_bitwise_equal(g["C"], O.os2_dgemm(A, B, 8)["C"], "C against the oracle")


def test_persistent_complex(monkeypatch):
    from test_gpu_zgemm import complex_case, run_complex
    A, B = complex_case(530, 280, 400, 7)
    monkeypatch.setenv("OZ2_GEMM_TILE", "256")
    monkeypatch.setenv("OZ2_GEMM_KERNEL", "blocks")
    g0 = run_complex(A, B, 14, want_prod=False)
    monkeypatch.setenv("OZ2_GEMM_KERNEL", "persistent")
    g1 = run_complex(A, B, 14, want_prod=False)
    assert np.array_equal(g1["red"], g0["red"]), "reduced planes differ"
    assert_bitwise_equal(g1["C_re"], g0["C_re"], "Re C")
    assert_bitwise_equal(g1["C_im"], g0["C_im"], "Im C")


def _walking_cases(seed=7201, count=8):
    # more 256 x 256 tiles than compute units (5 x 5 x 11 = 275 at the least),
    # ragged edges, padded leading dimensions, both modes
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        m, n = (int(x) for x in rng.integers(1030, 1301, size=2))
        k = int(rng.integers(250, 1100))
        N = int(rng.integers(11, 21))
        mode = "accurate" if rng.random() < 0.3 else "fast"
        pads = [int(x) for x in rng.integers(0, 4, size=3)]
        out.append((m, n, k, N, mode, pads, int(rng.integers(1 << 30))))
    return out


@pytest.mark.parametrize("m,n,k,N,mode,pads,seed", _walking_cases(),
                         ids=lambda v: None if not isinstance(v, tuple) else str(v))
def test_persistent_random_shapes_against_oracle(m, n, k, N, mode, pads, seed):
    assert -(-m // 256) * -(-n // 256) * N > 256  # the persistent kernel by default
    A, B = W.spread_case(m, n, k, 1.0, seed=seed)
    full_parity(A, B, N, mode, lda=m + pads[0], ldb=k + pads[1], ldc=m + pads[2], want_prod=False)

