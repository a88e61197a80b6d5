"""Register and scratch use of the INT8 GEMM kernels, from the compiler's
resource remarks for gfx950 (a device-only compile, no GPU needed), and the
persistent GEMM's M0 discipline in its compiled code.

The GEMM loops keep every accumulator and fragment in registers; a spill
would put scratch loads into the loop or the epilogue, and a scratch load's
counter wait also waits for every copy in flight. The persistent kernel runs
one wavefront per SIMD with all 512 registers in use, so this guards it
against a change that tips the allocation over."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _remarks():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    src = os.path.join(ROOT, "rns_emulated_fp64_amd", "csrc", "kernels.hip")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "--cuda-device-only", "-c",
           "-Rpass-analysis=kernel-resource-usage", src, "-o", os.devnull]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    kernels, cur = {}, None
    for line in out.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]+\])?: (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def kernels():
    return _remarks()


def _gemm_kernels(kernels):
    return {k: v for k, v in kernels.items() if "k_gemm" in k}


def test_gemm_kernels_found(kernels):
    names = _gemm_kernels(kernels)
    assert any("k_gemm_persistent" in k for k in names), sorted(kernels)
    assert any("k_gemm_crt" in k for k in names), sorted(kernels)
    assert sum("6k_gemmILi" in k for k in names) >= 3, sorted(names)  # EPI_MOD / EPI_RAW / EPI_BOUND


def test_gemm_kernels_do_not_spill(kernels):
    for name, r in _gemm_kernels(kernels).items():
        assert r.get("VGPRs Spill", 0) == 0, (name, r)
        assert r.get("ScratchSize", 0) == 0, (name, r)


def test_no_kernel_uses_scratch(kernels):
    # every kernel of the library (scale, split, GEMMs, reconstructions,
    # checks) keeps its state in registers and LDS
    assert len(kernels) > 20, sorted(kernels)
    for name, r in kernels.items():
        assert r.get("VGPRs Spill", 0) == 0 and r.get("ScratchSize", 0) == 0, (name, r)


def test_persistent_kernel_resources(kernels):
    name = next(k for k in kernels if "k_gemm_persistent" in k)
    r = kernels[name]
    assert r.get("SGPRs Spill", 0) == 0, r
    assert r["LDS Size"] == 5 * 32 * 1024, r  # the five-slot ring of 32 KiB stages
    assert r["Occupancy"] == 1, r             # one wavefront per SIMD by design


def test_persistent_kernel_m0_written_only_by_its_copies():
    # the persistent GEMM sets M0 (the LDS address of a copy) in one inline-asm
    # statement and issues the copy in the next; that is only sound if the
    # compiler writes M0 nowhere in the kernel itself
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    src = os.path.join(ROOT, "rns_emulated_fp64_amd", "csrc", "kernels.hip")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "--cuda-device-only", "-S", src,
           "-o", "-"]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = out.stdout.splitlines()
    start = next(i for i, l in enumerate(lines) if re.match(r"^_ZN3oz217k_gemm_persistent\S*:", l))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    in_asm, asm_writes, other = False, 0, []
    for l in lines[start:end]:
        t = l.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
        elif t.startswith(";;#ASMEND"):
            in_asm = False
        elif re.match(r"^s_\w+\s+m0\b", t):
            if in_asm:
                asm_writes += 1
            else:
                other.append(t)
    assert asm_writes >= 8, asm_writes
    assert not other, other
