"""Seeded synthetic inputs for the Ozaki Scheme II FP64 GEMM emulation.

This module holds random draws only, none of the method's arithmetic. The CPU
oracle (``oracle/``), the GPU parity tests and ``bench.py`` all take their
operands from here, so every side sees the same bits.

The shapes follow the pages' own experiments:
- random matrices whose entries spread over a range of exponents controlled by
  a parameter phi, with inner dimension k in {1024, 16384}
  ("Improved Scaling for Fast Mode of Ozaki Scheme II", section Ergebnisse);
- 16384 x 16384 products with 14 moduli ("8ビットの整数で53ビットの倍精度を
  組み立てる。中国剰余定理をGPUに載せたOzaki Scheme II", section
  行列積の回数と性能);
- ones matrices and uniform matrices multiplied by a power of two alpha, used
  to probe scale invariance ("Improved Scaling ...", section Problemstellung).

No public dataset is involved: the pages' workloads are themselves synthetic.

Conventions
-----------
Every generator returns numpy float64 arrays ``A`` of shape (m, k) and ``B`` of
shape (k, n) in natural mathematical orientation (``make`` rounds them to
binary32 for the single-precision workload). Random numbers are drawn
with ``numpy.random.default_rng(seed)`` (PCG64), A's arrays first and then B's,
each in C order. Callers convert to column-major storage themselves.
"""
from __future__ import annotations

import numpy as np


def spread_matrix(rng: np.random.Generator, shape, phi: float) -> np.ndarray:
    """Entries (U(0,1) - 0.5) * exp(phi * N(0,1)): phi sets the exponent spread.

    U is drawn first, then Z, both of the full shape.
    """
    u = rng.random(shape)
    z = rng.standard_normal(shape)
    return (u - 0.5) * np.exp(phi * z)


def uniform_case(m: int, n: int, k: int, seed: int = 0):
    """A, B with iid U(-1, 1) entries."""
    rng = np.random.default_rng(seed)
    a = rng.uniform(-1.0, 1.0, (m, k))
    b = rng.uniform(-1.0, 1.0, (k, n))
    return a, b


def spread_case(m: int, n: int, k: int, phi: float, seed: int = 0):
    """A, B with entries (U - 0.5) * exp(phi * Z); A drawn before B."""
    rng = np.random.default_rng(seed)
    a = spread_matrix(rng, (m, k), phi)
    b = spread_matrix(rng, (k, n), phi)
    return a, b


def scale_sweep_case(size: int = 2048, seed: int = 0):
    """Base operands of the scale-invariance sweep.

    Returns (ones_A, uniform_A, B): A is later multiplied by alpha = 2**s with
    ``numpy.ldexp`` (exact). U_A is drawn before B.
    """
    rng = np.random.default_rng(seed)
    ua = rng.uniform(-1.0, 1.0, (size, size))
    b = rng.uniform(-1.0, 1.0, (size, size))
    return np.ones((size, size)), ua, b


#: The workloads: name -> (m, n, k, N moduli, generator kwargs).
CONFIGS = {
    # 64^3, U(-1,1), N=8, fast mode: small enough for the oracle in well under a second.
    "u64_n8": dict(m=64, n=64, k=64, num_moduli=8, kind="uniform", seed=0),
    # 1024^3, moderate exponent spread phi=0.5, N=14.
    "spread0.5_1024_n14": dict(m=1024, n=1024, k=1024, num_moduli=14, kind="spread", phi=0.5, seed=0),
    # 4096^3, wide exponent spread phi=1.0, N=16: the headline workload.
    "spread1.0_4096_n16": dict(m=4096, n=4096, k=4096, num_moduli=16, kind="spread", phi=1.0, seed=0),
    # 512^3, phi=1.0, N=14: a small product (the GEMM's 128 x 128 block shape).
    "spread1.0_512_n14": dict(m=512, n=512, k=512, num_moduli=14, kind="spread", phi=1.0, seed=0),
    # 256^3, phi=1.0, N=14: a launch-bound product (one- vs two-launch steps 3-5).
    "spread1.0_256_n14": dict(m=256, n=256, k=256, num_moduli=14, kind="spread", phi=1.0, seed=0),
    # 2048^3 scale sweep, N=14.
    "scale_sweep_2048_n14": dict(m=2048, n=2048, k=2048, num_moduli=14, kind="sweep", seed=0),
    # 2048^3 and 8192^3, phi=1.0, N=16: the headline draw at the sizes around it
    # (a size sweep of the GEMM kernels).
    "spread1.0_2048_n16": dict(m=2048, n=2048, k=2048, num_moduli=16, kind="spread", phi=1.0, seed=0),
    "spread1.0_8192_n16": dict(m=8192, n=8192, k=8192, num_moduli=16, kind="spread", phi=1.0, seed=0),
    # 16384^3, phi=1.0, N=18 (2 GiB per operand).
    "spread1.0_16384_n18": dict(m=16384, n=16384, k=16384, num_moduli=18, kind="spread", phi=1.0, seed=0),
    # Single precision ("Improved Scaling ...", section Zentrale Beiträge: the
    # scheme is also evaluated for SGEMM): the phi=1.0 draw at 4096^3 rounded
    # to binary32, N=8.
    "sgemm_spread1.0_4096_n8": dict(m=4096, n=4096, k=4096, num_moduli=8, kind="spread", phi=1.0, seed=0,
                                    single=True),
    # Complex products ("Improved Scaling ...", closing remark: ZGEMM/CGEMM):
    # real and imaginary parts drawn like the phi=1.0 workload at 4096^3, N=16.
    "zgemm_spread1.0_4096_n16": dict(m=4096, n=4096, k=4096, num_moduli=16, kind="spread", phi=1.0, seed=0,
                                     complex=True),
}


def complex_spread_case(m: int, n: int, k: int, phi: float, seed: int = 0):
    """Complex A, B: Re A, Im A, Re B, Im B drawn in that order as spread_matrix."""
    rng = np.random.default_rng(seed)
    ar, ai = spread_matrix(rng, (m, k), phi), spread_matrix(rng, (m, k), phi)
    br, bi = spread_matrix(rng, (k, n), phi), spread_matrix(rng, (k, n), phi)
    return ar + 1j * ai, br + 1j * bi


def make(name: str):
    """Operands (A, B) of a named workload (not for the scale sweep); binary32
    arrays (the float64 draw rounded to nearest) for single-precision ones."""
    c = CONFIGS[name]
    if c.get("complex"):
        return complex_spread_case(c["m"], c["n"], c["k"], c["phi"], c["seed"])
    if c["kind"] == "uniform":
        a, b = uniform_case(c["m"], c["n"], c["k"], c["seed"])
    elif c["kind"] == "spread":
        a, b = spread_case(c["m"], c["n"], c["k"], c["phi"], c["seed"])
    else:
        raise ValueError(f"{name} is a sweep; use scale_sweep_case()")
    if c.get("single"):
        return a.astype(np.float32), b.astype(np.float32)
    return a, b
