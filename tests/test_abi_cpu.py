"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, validates arguments before touching the device, and its own
tables agree with the oracle's independently built ones."""
import math
import os
import re

import pytest

import oracle as O
import rns_emulated_fp64_amd as oz

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ozaki2.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ozaki2_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    L = oz.lib()
    names = declared_functions()
    assert len(names) >= 10
    assert sorted(oz.EXPORTS) == names
    for name in names:
        assert hasattr(L, name), name


def test_nm_lists_symbols():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", oz.LIB_PATH], capture_output=True, text=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_no_library_symbol_left_undefined():
    # every kernel launch stub and helper of the library is defined in it (a
    # kernel template whose host stub the compiler dropped shows up here)
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", oz.LIB_PATH], capture_output=True, text=True).stdout
    assert "oz2" not in out, [l for l in out.splitlines() if "oz2" in l][:4]


def test_check_entry_host_checks():
    assert oz.ozaki2_check_workspace_size(64, 64, 64, 20, 0) == 0  # no 21st modulus
    assert oz.ozaki2_check_workspace_size(64, 64, 64, 16, 0) > oz.ozaki2_workspace_size(64, 64, 64, 16, 0)
    need = oz.ozaki2_check_workspace_size(64, 64, 64, 16, 0)
    assert oz.ozaki2_dgemm_check(64, 64, 64, P, 64, P, 64, P, 64, 20, 0, P, need, P, 0) == -10
    assert oz.ozaki2_dgemm_check(64, 64, 64, P, 64, P, 64, P, 64, 16, 0, P, need, 0, 0) == -14
    assert oz.ozaki2_dgemm_check(64, 64, 64, P, 64, P, 64, P, 64, 16, 0, P + 64, need, P, 0) == -12
    assert oz.ozaki2_dgemm_check(64, 64, 64, P, 64, P, 64, P, 64, 16, 0, P, need - 1, P, 0) == 2
    assert oz.ozaki2_crt_check_debug(4, 4, 20, P, P, P, P, 4, P, P, 1 << 40, 0) == -3
    assert oz.ozaki2_crt_check_debug(4, 4, 8, P, P, P, P, 4, 0, P, 1 << 40, 0) == -9
    assert oz.ozaki2_crt_check_debug(4, 4, 8, P, P, P, P, 4, P, P + 8, 1 << 40, 0) == -10
    assert oz.ozaki2_crt_check_debug(4, 4, 8, P, P, P, P, 4, P, P, 16, 0) == 2


def test_noalloc_host_checks():
    # argument errors and the array limit come back before any HIP call
    assert oz.ozaki2_dgemm_noalloc(-1, 4, 4, P, 4, P, 4, P, 4, 8, 0, 0) == -1
    assert oz.ozaki2_dgemm_noalloc(4, 4, 4, P, 4, P, 4, P, 4, 1, 0, 0) == -10
    assert oz.ozaki2_dgemm_noalloc(0, 4, 4, P, 1, P, 4, P, 1, 8, 0, 0) == 0
    assert oz.ozaki2_dgemm_noalloc(4096, 4096, 4096, P, 4096, P, 4096, P, 4096, 16, 0, 0) == oz.ERR_NOALLOC_LIMIT
    assert "noalloc" in oz.status_string(oz.ERR_NOALLOC_LIMIT)
    # the header's limit is the binding's
    text = open(HEADER).read()
    assert "#define OZAKI2_NOALLOC_MAX_WORKSPACE (128u << 20)" in text
    assert oz.NOALLOC_MAX_WORKSPACE == 128 << 20


def test_moduli_and_constants_match_oracle():
    assert oz.ozaki2_max_moduli() == 20
    for n in range(2, 21):
        mods = oz.ozaki2_moduli(n)
        assert mods == O.choose_moduli(n)
        t = O.crt_tables(mods)
        assert oz.ozaki2_scaling_constant(n) == O.scaling_constant(t["P"]), n
        for l in range(n):
            assert oz.ozaki2_crt_weight(n, l) == t["W"][l]


def test_host_argument_errors():
    L = oz.lib()
    with pytest.raises(oz.Ozaki2Error):
        oz.ozaki2_moduli(0)
    with pytest.raises(oz.Ozaki2Error):
        oz.ozaki2_scaling_constant(21)
    assert L.ozaki2_moduli(3, None) == -2
    assert L.ozaki2_crt_weight(8, 8, None, 8) == -2


P = 1 << 20  # a fake non-null pointer: validation fails before it is ever used


@pytest.mark.parametrize(
    "args,status",
    [
        ((-1, 4, 4, P, 4, P, 4, P, 4, 8, 0), -1),
        ((4, -1, 4, P, 4, P, 4, P, 4, 8, 0), -2),
        ((4, 4, -1, P, 4, P, 4, P, 4, 8, 0), -3),
        ((4, 4, 4, 0, 4, P, 4, P, 4, 8, 0), -4),
        ((4, 4, 4, P, 3, P, 4, P, 4, 8, 0), -5),
        ((4, 4, 4, P, 4, 0, 4, P, 4, 8, 0), -6),
        ((4, 4, 4, P, 4, P, 3, P, 4, 8, 0), -7),
        ((4, 4, 4, P, 4, P, 4, 0, 4, 8, 0), -8),
        ((4, 4, 4, P, 4, P, 4, P, 3, 8, 0), -9),
        ((4, 4, 4, P, 4, P, 4, P, 4, 1, 0), -10),
        ((4, 4, 4, P, 4, P, 4, P, 4, 21, 0), -10),
        ((4, 4, 4, P, 4, P, 4, P, 4, 8, 3), -11),
        ((4, 4, 4, P, 4, P, 4, P, 4, 8, -1), -11),
        ((4, 4, 1 << 22, P, 4, P, 1 << 22, P, 4, 8, 0), 3),
        ((4, 4, 1 << 19, P, 4, P, 1 << 19, P, 4, 8, 1), 3),
        # quick returns: nothing is launched for an empty C
        ((0, 4, 4, 0, 1, P, 4, 0, 1, 8, 0), 0),
        ((4, 0, 4, P, 4, 0, 4, 0, 4, 8, 0), 0),
    ],
)
def test_status_codes(args, status):
    assert oz.ozaki2_dgemm(*args, 0) == status
    assert oz.ozaki2_dgemm_ws(*args, P, 1 << 40, 0) == status
    assert oz.ozaki2_sgemm(*args, 0) == status
    assert oz.ozaki2_sgemm_ws(*args, P, 1 << 40, 0) == status


def test_complex_status_codes():
    # same argument checks as the real entry points; accurate mode is not defined for complex products
    for fn in (oz.ozaki2_zgemm, oz.ozaki2_cgemm):
        assert fn(-1, 4, 4, P, 4, P, 4, P, 4, 8, 0, 0) == -1
        assert fn(4, 4, 4, P, 3, P, 4, P, 4, 8, 0, 0) == -5
        assert fn(4, 4, 4, P, 4, P, 4, P, 4, 21, 0, 0) == -10
        assert fn(4, 4, 4, P, 4, P, 4, P, 4, 8, 1, 0) == 3
        assert fn(4, 4, 4, P, 4, P, 4, P, 4, 8, 2, 0) == 3
        assert fn(0, 4, 4, 0, 1, P, 4, 0, 1, 8, 0, 0) == 0
    assert oz.ozaki2_zgemm_ws(4, 4, 4, P, 4, P, 4, P, 4, 8, 0, 0, 0, 0) == -12
    need = oz.ozaki2_zgemm_workspace_size(64, 64, 64, 8)
    assert need > oz.ozaki2_workspace_size(64, 64, 64, 8, 0)
    assert oz.ozaki2_zgemm_ws(64, 64, 64, P, 64, P, 64, P, 64, 8, 0, P, need - 1, 0) == 2
    assert oz.ozaki2_zgemm_workspace_size(64, 64, 64, 8, debug=True) > need


def test_workspace_checks():
    assert oz.ozaki2_dgemm_ws(64, 64, 64, P, 64, P, 64, P, 64, 8, 0, 0, 0, 0) == -12
    need = oz.ozaki2_workspace_size(64, 64, 64, 8, 0)
    assert need > 0
    assert oz.ozaki2_dgemm_ws(64, 64, 64, P, 64, P, 64, P, 64, 8, 0, P, need - 1, 0) == 2
    # the workspace must be 256-byte aligned (-12, before any HIP call)
    for off in (8, 16, 128):
        assert oz.ozaki2_dgemm_ws(64, 64, 64, P, 64, P, 64, P, 64, 8, 0, P + off, need, 0) == -12
        assert oz.ozaki2_sgemm_ws(64, 64, 64, P, 64, P, 64, P, 64, 8, 0, P + off, need, 0) == -12
        assert oz.ozaki2_crt_debug(4, 4, 8, P, P, P, P, 4, P + off, 1 << 40, 0) == -9
    assert oz.ozaki2_workspace_size(0, 4, 4, 8, 0) == 0
    assert oz.ozaki2_workspace_size(4, 4, 4, 1, 0) == 0
    # residues dominate: N * (m_pad + n_pad) * k_pad + N * m_pad * n_pad bytes
    ws = oz.ozaki2_workspace_size(4096, 4096, 4096, 16, 0)
    assert 16 * (2 * 4096 * 4096 + 4096 * 4096) <= ws < 16 * 3 * 4096 * 4096 * 1.05
    assert oz.ozaki2_workspace_size(4096, 4096, 4096, 16, 1) > ws
    assert oz.ozaki2_debug_workspace_size(300, 200, 500, 8, 0) > oz.ozaki2_workspace_size(300, 200, 500, 8, 0)


@pytest.mark.parametrize(
    "args,status",
    [
        ((-1, 4, 8, P, P, P, P, 4, P, 1 << 40), -1),
        ((4, -1, 8, P, P, P, P, 4, P, 1 << 40), -2),
        ((4, 4, 1, P, P, P, P, 4, P, 1 << 40), -3),
        ((4, 4, 21, P, P, P, P, 4, P, 1 << 40), -3),
        ((4, 4, 8, 0, P, P, P, 4, P, 1 << 40), -4),
        ((4, 4, 8, P, 0, P, P, 4, P, 1 << 40), -5),
        ((4, 4, 8, P, P, 0, P, 4, P, 1 << 40), -6),
        ((4, 4, 8, P, P, P, 0, 4, P, 1 << 40), -7),
        ((4, 4, 8, P, P, P, P, 3, P, 1 << 40), -8),
        ((4, 4, 8, P, P, P, P, 4, 0, 1 << 40), -9),
        ((4, 4, 8, P, P, P, P, 4, P, 16), 2),
        ((1 << 31, 4, 8, P, P, P, P, 1 << 31, P, 1 << 60), 3),
        ((0, 4, 8, 0, 0, 0, 0, 1, 0, 0), 0),
    ],
)
def test_crt_debug_status_codes(args, status):
    assert oz.ozaki2_crt_debug(*args, 0) == status


def test_status_strings():
    for s in (0, 1, 2, 3, -4, 99):
        assert isinstance(oz.status_string(s), str) and oz.status_string(s)


def test_timing_off_and_empty_read_need_no_device():
    # turning timing off and reading an empty record touch no HIP call
    oz.ozaki2_timing_enable(0)
    ms, calls = oz.ozaki2_timing_read()
    assert calls == 0 and ms == {p: 0.0 for p in oz.PHASES}
    assert oz.ozaki2_timing_read_calls(0) == []


def test_bench_refuses_more_than_one_gpu():
    # the benchmark measures one GPU; asking for more exits with a message
    # before anything touches a device
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
