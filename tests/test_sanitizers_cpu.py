"""Address and undefined-behaviour sanitizer builds of the native host code
(no GPU): the oracle's C core (gcc) and the library's table construction
(tables.cpp, g++), each linked with a small driver that runs every function
over its edge cases and checks a few results; any sanitizer report fails the
run (-fno-sanitize-recover=all) and so the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

ORACLE_DRIVER = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
int orc_split(int64_t, int64_t, const double *, int64_t, int64_t, const int32_t *, int, const int32_t *, int8_t *);
int orc_scaled_ints(int64_t, int64_t, const double *, int64_t, int64_t, const int32_t *, int64_t *, int64_t *);
void orc_dd_gemm(int64_t, int64_t, int64_t, const double *, int64_t, const double *, int64_t, double *, double *);
static int mod_pow2(int e, int p) { int r = 1 % p; for (int i = 0; i < e; ++i) r = (r * 2) % p; return r; }
int main(void) {
    const int32_t mods[4] = {256, 255, 253, 251};
    /* rows: 2^100, -2^100 + 2^48, 0, a subnormal, 1.5, -7.25; scaled by 2^0 except row 4 */
    double X[6 * 2] = {0x1p100, 3.0, -0x1p100 + 0x1p48, -1.0, 0.0, 0.0, 0x1p-1070, 0x1p-1074, 1.5, -2.5, -7.25, 7.75};
    int32_t e[6] = {0, 0, 0, 1100, 3, 2};
    int8_t out[4 * 6 * 2];
    if (orc_split(6, 2, X, 2, 1, e, 4, mods, out) != 0) return 10;
    for (int l = 1; l < 4; ++l) {  /* 2^100 mod p, symmetric */
        int p = mods[l], r = mod_pow2(100, p);
        if (r > (p - 1) / 2) r -= p;
        if (out[(l * 6 + 0) * 2 + 0] != r) return 11;
    }
    if (out[(0 * 6 + 5) * 2 + 0] != -29) return 12;  /* trunc(-7.25 * 4) = -29 mod 256 */
    int64_t hi[12], lo[12];
    if (orc_scaled_ints(6, 2, X, 2, 1, e, hi, lo) != 0) return 13;
    double bad[2] = {INFINITY, 1.0};
    int32_t e0[1] = {0};
    if (orc_split(1, 2, bad, 2, 1, e0, 4, mods, out) != -1) return 14;
    double big[1] = {0x1p126};
    if (orc_scaled_ints(1, 1, big, 1, 1, e0, hi, lo) != -1) return 15;
    /* double-double product of small integers is exact */
    double A[6] = {1, 2, 3, 4, 5, 6}, B[6] = {1, -1, 2, 0, 3, 1}, chi[4], clo[4];
    orc_dd_gemm(2, 2, 3, A, 2, B, 3, chi, clo);  /* A 2x3 (lda 2), B 3x2 (ldb 3), column-major */
    const double want[4] = {8, 10, 14, 18};  /* A = [1 3 5; 2 4 6], B = [1 0; -1 3; 2 1] */
    for (int i = 0; i < 4; ++i)
        if (chi[i] != want[i] || clo[i] != 0.0) return 16;
    printf("oracle core ok\n");
    return 0;
}
"""

TABLES_DRIVER = r"""
#include "tables.h"
#include <cstdio>
using namespace oz2;
static uint32_t limbs_mod(const uint32_t *w, int limbs, uint32_t p) {
    uint64_t r = 0;
    for (int i = limbs - 1; i >= 0; --i) r = ((r << 32) | w[i]) % p;
    return (uint32_t)r;
}
int main() {
    const int32_t want[20] = {256, 255, 253, 251, 247, 241, 239, 233, 229, 227,
                              223, 217, 211, 199, 197, 193, 191, 181, 179, 173};
    int32_t got[20];
    if (!greedy_moduli(20, got) || greedy_moduli(21, got) || greedy_moduli(0, got)) return 10;
    for (int i = 0; i < 20; ++i)
        if (got[i] != want[i]) return 11;
    if (get_tables(1) != nullptr || get_tables(21) != nullptr) return 12;
    double last = 0.0;
    for (int n = 2; n <= 20; ++n) {
        const Tables *t = get_tables(n);
        if (!t || t->n != n || !(t->Pp > last)) return 13;
        last = t->Pp;
        for (int l = 0; l < n; ++l)        /* the weights advance one clock only */
            for (int i = 0; i < n; ++i)
                if (limbs_mod(t->weight[l], t->weight_limbs, (uint32_t)t->moduli[i]) != (l == i ? 1u : 0u)) return 14;
        if (n < 20) {
            if (t->check.pc != want[n]) return 15;
            for (int l = 0; l < n; ++l)
                if ((uint32_t)t->check.wm[l] != limbs_mod(t->weight[l], t->weight_limbs, (uint32_t)want[n])) return 16;
        }
    }
    std::printf("tables ok\n");
    return 0;
}
"""


def _build_and_run(tmp_path, compiler, src_name, driver, sources, extra):
    drv = tmp_path / src_name
    drv.write_text(driver)
    exe = tmp_path / (src_name + ".bin")
    cmd = [compiler, *SAN, *extra, str(drv), *sources, "-o", str(exe), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.returncode, run.stdout[-2000:], run.stderr[-3000:])
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-3000:]
    return run.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_core_under_asan_ubsan(tmp_path):
    out = _build_and_run(tmp_path, "gcc", "oracle_driver.c", ORACLE_DRIVER,
                         [os.path.join(ROOT, "oracle", "oracle_core.c")], ["-std=gnu11", "-ffp-contract=off"])
    assert "oracle core ok" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not installed")
def test_host_tables_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "rns_emulated_fp64_amd", "csrc")
    out = _build_and_run(tmp_path, "g++", "tables_driver.cpp", TABLES_DRIVER, [os.path.join(csrc, "tables.cpp")],
                         ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + csrc,
                          "-I" + os.path.join(ROOT, "include")])
    assert "tables ok" in out
