"""CPU oracle for the Ozaki Scheme II GEMM emulation -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
import this package. The library in rns_emulated_fp64_amd/ never does, and
shares no code with it.
"""
from .ozaki2_oracle import *  # noqa: F401,F403
from .ozaki2_oracle import build_core  # noqa: F401
