"""Python binding of libozaki2: FP64 matrix products emulated by Ozaki Scheme II
on the INT8 matrix cores of MI355X (gfx950).

Argument marshalling only: every step of the product runs in the HIP kernels
of ``libozaki2.so`` (built in-tree by ``python -m rns_emulated_fp64_amd.build``).
There is no CPU fallback; loading fails loudly when the library is missing.

Functions named like the C ABI (``ozaki2_dgemm`` ...) take plain integers and
device pointers exactly as ``include/ozaki2.h`` documents. ``dgemm`` is the
convenience form on torch tensors (torch provides device memory and streams).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libozaki2.so")

FAST = 0
ACCURATE = 1
ERR_NOALLOC_LIMIT = 4  # OZAKI2_ERR_NOALLOC_LIMIT
NOALLOC_MAX_WORKSPACE = 128 << 20  # OZAKI2_NOALLOC_MAX_WORKSPACE
FAST_ORIGINAL = 2  # comparison stand-in for the original fast-mode rule (see include/ozaki2.h)
MODES = {"fast": FAST, "accurate": ACCURATE, "original": FAST_ORIGINAL}
PHASES = ("scale", "split", "gemm", "crt")

#: every symbol include/ozaki2.h declares
EXPORTS = (
    "ozaki2_dgemm", "ozaki2_workspace_size", "ozaki2_dgemm_ws", "ozaki2_dgemm_debug",
    "ozaki2_debug_workspace_size", "ozaki2_max_moduli", "ozaki2_moduli", "ozaki2_scaling_constant",
    "ozaki2_crt_weight", "ozaki2_status_string", "ozaki2_timing_enable", "ozaki2_timing_read",
    "ozaki2_timing_read_calls",
    "ozaki2_finalize", "ozaki2_crt_debug", "ozaki2_sgemm", "ozaki2_sgemm_ws", "ozaki2_sgemm_debug",
    "ozaki2_zgemm", "ozaki2_zgemm_ws", "ozaki2_zgemm_debug", "ozaki2_cgemm", "ozaki2_cgemm_ws", "ozaki2_cgemm_debug",
    "ozaki2_zgemm_workspace_size", "ozaki2_dgemm_noalloc", "ozaki2_dgemm_check", "ozaki2_check_workspace_size",
    "ozaki2_crt_check_debug", "ozaki2_zcrt_debug",
)

_lib = None


class Ozaki2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libozaki2.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m rns_emulated_fp64_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, p, i32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    prod = [i64, i64, i64, p, i64, p, i64, p, i64, i32, i32]
    L.ozaki2_dgemm.argtypes = prod + [p]
    L.ozaki2_dgemm.restype = i32
    L.ozaki2_dgemm_noalloc.argtypes = prod + [p]
    L.ozaki2_dgemm_noalloc.restype = i32
    L.ozaki2_workspace_size.argtypes = [i64, i64, i64, i32, i32]
    L.ozaki2_workspace_size.restype = sz
    L.ozaki2_debug_workspace_size.argtypes = [i64, i64, i64, i32, i32]
    L.ozaki2_debug_workspace_size.restype = sz
    L.ozaki2_dgemm_ws.argtypes = prod + [p, sz, p]
    L.ozaki2_dgemm_ws.restype = i32
    L.ozaki2_dgemm_debug.argtypes = prod + [p, sz, p, p, p, p, p, p, p]
    L.ozaki2_dgemm_debug.restype = i32
    for prefix in ("ozaki2_sgemm", "ozaki2_zgemm", "ozaki2_cgemm"):
        for suffix in ("", "_ws", "_debug"):
            getattr(L, prefix + suffix).argtypes = getattr(L, "ozaki2_dgemm" + suffix).argtypes
            getattr(L, prefix + suffix).restype = i32
    L.ozaki2_zgemm_workspace_size.argtypes = [i64, i64, i64, i32, i32]
    L.ozaki2_zgemm_workspace_size.restype = sz
    L.ozaki2_crt_debug.argtypes = [i64, i64, i32, p, p, p, p, i64, p, sz, p]
    L.ozaki2_crt_debug.restype = i32
    L.ozaki2_zcrt_debug.argtypes = L.ozaki2_crt_debug.argtypes
    L.ozaki2_zcrt_debug.restype = i32
    L.ozaki2_dgemm_check.argtypes = prod + [p, sz, p, p]
    L.ozaki2_dgemm_check.restype = i32
    L.ozaki2_check_workspace_size.argtypes = [i64, i64, i64, i32, i32]
    L.ozaki2_check_workspace_size.restype = sz
    L.ozaki2_crt_check_debug.argtypes = [i64, i64, i32, p, p, p, p, i64, p, p, sz, p]
    L.ozaki2_crt_check_debug.restype = i32
    L.ozaki2_max_moduli.argtypes = []
    L.ozaki2_max_moduli.restype = i32
    L.ozaki2_moduli.argtypes = [i32, p]
    L.ozaki2_moduli.restype = i32
    L.ozaki2_scaling_constant.argtypes = [i32, p]
    L.ozaki2_scaling_constant.restype = i32
    L.ozaki2_crt_weight.argtypes = [i32, i32, p, i32]
    L.ozaki2_crt_weight.restype = i32
    L.ozaki2_status_string.argtypes = [i32]
    L.ozaki2_status_string.restype = ctypes.c_char_p
    L.ozaki2_timing_enable.argtypes = [i32, i32]
    L.ozaki2_timing_enable.restype = i32
    L.ozaki2_timing_read.argtypes = [p, p]
    L.ozaki2_timing_read.restype = i32
    L.ozaki2_timing_read_calls.argtypes = [p, i32, p]
    L.ozaki2_timing_read_calls.restype = i32
    L.ozaki2_finalize.argtypes = []
    L.ozaki2_finalize.restype = None
    _lib = L
    return L


# ---- same names as the C ABI: plain integers / device pointers ----------------
def ozaki2_dgemm(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, stream=0) -> int:
    return lib().ozaki2_dgemm(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, stream)


def ozaki2_dgemm_noalloc(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, stream=0) -> int:
    return lib().ozaki2_dgemm_noalloc(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, stream)


def ozaki2_dgemm_check(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes, flags,
                       stream=0) -> int:
    return lib().ozaki2_dgemm_check(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                                    flags, stream)


def ozaki2_check_workspace_size(m, n, k, num_moduli, mode) -> int:
    return lib().ozaki2_check_workspace_size(m, n, k, num_moduli, mode)


def ozaki2_crt_check_debug(m, n, num_moduli, residues, e, f, C, ldc, flags, workspace, workspace_bytes,
                           stream=0) -> int:
    return lib().ozaki2_crt_check_debug(m, n, num_moduli, residues, e, f, C, ldc, flags, workspace, workspace_bytes,
                                        stream)


def ozaki2_workspace_size(m, n, k, num_moduli, mode) -> int:
    return lib().ozaki2_workspace_size(m, n, k, num_moduli, mode)


def ozaki2_debug_workspace_size(m, n, k, num_moduli, mode) -> int:
    return lib().ozaki2_debug_workspace_size(m, n, k, num_moduli, mode)


def ozaki2_dgemm_ws(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes, stream=0) -> int:
    return lib().ozaki2_dgemm_ws(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace,
                                 workspace_bytes, stream)


def ozaki2_dgemm_debug(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                       e_out, f_out, resA_out, resB_out, prod_out, red_out, stream=0) -> int:
    return lib().ozaki2_dgemm_debug(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace,
                                    workspace_bytes, e_out, f_out, resA_out, resB_out, prod_out, red_out, stream)


def ozaki2_sgemm(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, stream=0) -> int:
    return lib().ozaki2_sgemm(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, stream)


def ozaki2_sgemm_ws(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes, stream=0) -> int:
    return lib().ozaki2_sgemm_ws(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                                 stream)


def ozaki2_sgemm_debug(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                       e_out, f_out, resA_out, resB_out, prod_out, red_out, stream=0) -> int:
    return lib().ozaki2_sgemm_debug(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                                    e_out, f_out, resA_out, resB_out, prod_out, red_out, stream)


def ozaki2_zgemm(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode=FAST, stream=0) -> int:
    return lib().ozaki2_zgemm(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, stream)


def ozaki2_zgemm_ws(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes, stream=0) -> int:
    return lib().ozaki2_zgemm_ws(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                                 stream)


def ozaki2_zgemm_debug(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                       e_out, f_out, resA_out, resB_out, prod_out, red_out, stream=0) -> int:
    return lib().ozaki2_zgemm_debug(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                                    e_out, f_out, resA_out, resB_out, prod_out, red_out, stream)


def ozaki2_cgemm(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode=FAST, stream=0) -> int:
    return lib().ozaki2_cgemm(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, stream)


def ozaki2_cgemm_ws(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes, stream=0) -> int:
    return lib().ozaki2_cgemm_ws(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                                 stream)


def ozaki2_cgemm_debug(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                       e_out, f_out, resA_out, resB_out, prod_out, red_out, stream=0) -> int:
    return lib().ozaki2_cgemm_debug(m, n, k, A, lda, B, ldb, C, ldc, num_moduli, mode, workspace, workspace_bytes,
                                    e_out, f_out, resA_out, resB_out, prod_out, red_out, stream)


def ozaki2_zgemm_workspace_size(m, n, k, num_moduli, debug=False) -> int:
    return lib().ozaki2_zgemm_workspace_size(m, n, k, num_moduli, 1 if debug else 0)


def ozaki2_crt_debug(m, n, num_moduli, residues, e, f, C, ldc, workspace, workspace_bytes, stream=0) -> int:
    return lib().ozaki2_crt_debug(m, n, num_moduli, residues, e, f, C, ldc, workspace, workspace_bytes, stream)


def ozaki2_zcrt_debug(m, n, num_moduli, residues, e, f, C, ldc, workspace, workspace_bytes, stream=0) -> int:
    return lib().ozaki2_zcrt_debug(m, n, num_moduli, residues, e, f, C, ldc, workspace, workspace_bytes, stream)


def ozaki2_max_moduli() -> int:
    return lib().ozaki2_max_moduli()


def ozaki2_moduli(num_moduli: int) -> list[int]:
    out = (ctypes.c_int32 * max(num_moduli, 1))()
    st = lib().ozaki2_moduli(num_moduli, out)
    if st:
        raise Ozaki2Error(st, "ozaki2_moduli")
    return list(out)[:num_moduli]


def ozaki2_scaling_constant(num_moduli: int) -> float:
    out = ctypes.c_double()
    st = lib().ozaki2_scaling_constant(num_moduli, ctypes.byref(out))
    if st:
        raise Ozaki2Error(st, "ozaki2_scaling_constant")
    return out.value


def ozaki2_crt_weight(num_moduli: int, l: int) -> int:
    limbs = (ctypes.c_uint32 * 8)()
    used = lib().ozaki2_crt_weight(num_moduli, l, limbs, 8)
    if used < 0:
        raise Ozaki2Error(used, "ozaki2_crt_weight")
    return sum(int(limbs[i]) << (32 * i) for i in range(used))


def status_string(status: int) -> str:
    return lib().ozaki2_status_string(status).decode()


def ozaki2_timing_enable(max_calls: int, all_phases: bool = False) -> None:
    st = lib().ozaki2_timing_enable(max_calls, 1 if all_phases else 0)
    if st:
        raise Ozaki2Error(st, "ozaki2_timing_enable")


def ozaki2_timing_read() -> tuple[dict, int]:
    ms = (ctypes.c_double * 4)()
    calls = ctypes.c_int()
    st = lib().ozaki2_timing_read(ms, ctypes.byref(calls))
    if st:
        raise Ozaki2Error(st, "ozaki2_timing_read")
    return dict(zip(PHASES, list(ms))), calls.value


def ozaki2_timing_read_calls(max_calls: int) -> list:
    """Per timed call, a dict of milliseconds per phase; clears the record."""
    ms = (ctypes.c_double * (4 * max(max_calls, 1)))()
    calls = ctypes.c_int()
    st = lib().ozaki2_timing_read_calls(ms, max_calls, ctypes.byref(calls))
    if st:
        raise Ozaki2Error(st, "ozaki2_timing_read_calls")
    return [dict(zip(PHASES, list(ms[4 * c:4 * c + 4]))) for c in range(calls.value)]


def ozaki2_finalize() -> None:
    lib().ozaki2_finalize()


# ---- torch convenience -------------------------------------------------------
def _mode(mode) -> int:
    return MODES[mode] if isinstance(mode, str) else int(mode)


def dgemm(A, B, num_moduli: int = 16, mode="fast", out=None, workspace=None):
    """C = A @ B for float64 CUDA (HIP) tensors in row-major layout.

    Row-major C = A B is column-major C^T = B^T A^T, so the library is called
    with the operands swapped; the scaling is symmetric in the two operands.
    ``out`` (optional) must be a contiguous (m, n) tensor of the same dtype on
    the same device; ``workspace`` (optional) a device tensor of at least
    ``ozaki2_workspace_size`` bytes.
    """
    return _gemm(A, B, num_moduli, mode, out, workspace, "d")


def sgemm(A, B, num_moduli: int = 8, mode="fast", out=None, workspace=None):
    """C = A @ B for float32 CUDA (HIP) tensors (ozaki2_sgemm), as dgemm."""
    return _gemm(A, B, num_moduli, mode, out, workspace, "s")


def zgemm(A, B, num_moduli: int = 16, mode="fast", out=None, workspace=None):
    """C = A @ B for complex128 CUDA (HIP) tensors (ozaki2_zgemm, fast mode), as
    dgemm; a complex tensor's storage is the interleaved (re, im) layout the
    library takes. ``workspace`` needs ``ozaki2_zgemm_workspace_size`` bytes."""
    return _gemm(A, B, num_moduli, mode, out, workspace, "z")


def cgemm(A, B, num_moduli: int = 16, mode="fast", out=None, workspace=None):
    """C = A @ B for complex64 CUDA (HIP) tensors (ozaki2_cgemm), as zgemm."""
    return _gemm(A, B, num_moduli, mode, out, workspace, "c")


_KINDS = {  # dtype name, plain entry, workspace entry
    "d": ("float64", "ozaki2_dgemm"),
    "s": ("float32", "ozaki2_sgemm"),
    "z": ("complex128", "ozaki2_zgemm"),
    "c": ("complex64", "ozaki2_cgemm"),
}


def _gemm(A, B, num_moduli, mode, out, workspace, kind):
    import torch

    dname, entry = _KINDS[kind]
    dt = getattr(torch, dname)
    if A.dtype != dt or B.dtype != dt or not A.is_cuda or not B.is_cuda or A.device != B.device:
        raise TypeError(f"A and B must be {dt} tensors on the same GPU")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError("shapes do not multiply")
    A = A.contiguous()
    B = B.contiguous()
    m, k = A.shape
    n = B.shape[1]
    if out is None:
        C = torch.empty((m, n), dtype=dt, device=A.device)
    else:
        if out.dtype != dt or out.device != A.device or tuple(out.shape) != (m, n) or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous ({m}, {n}) {dt} tensor on {A.device}")
        C = out
    md = _mode(mode)
    plain, ws_form = globals()[entry], globals()[entry + "_ws"]
    if workspace is not None and (not workspace.is_cuda or workspace.device != A.device):
        raise ValueError(f"workspace must be a tensor on {A.device}")
    # the library launches on the current device: make it the operands' one
    with torch.cuda.device(A.device):
        stream = torch.cuda.current_stream(A.device).cuda_stream
        if workspace is None:
            st = plain(n, m, k, B.data_ptr(), max(n, 1), A.data_ptr(), max(k, 1), C.data_ptr(), max(n, 1),
                       num_moduli, md, stream)
        else:
            st = ws_form(n, m, k, B.data_ptr(), max(n, 1), A.data_ptr(), max(k, 1), C.data_ptr(), max(n, 1),
                         num_moduli, md, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                         stream)
    if st:
        raise Ozaki2Error(st, entry)
    return C
