"""Benchmark of the Ozaki Scheme II FP64 GEMM emulation on one MI355X.

One step = one ozaki2_dgemm_ws call (all phases: exponents, residue split,
INT8 GEMMs, CRT + unscale) on operands already resident in HBM. Prints ONE
JSON line. ``roofline`` rates the dominant kernel (the INT8 GEMM): its N*2mnk
int8 operations per launch over its average launch time, from HIP events on
the library's stream in the timed region, against the 5000 TOP/s dense INT8
peak; ``traffic`` is its HBM bytes per launch from the committed counter
record while the GEMM source still matches it. ``cpu_baseline`` times the CPU
oracle on the same workload (all rows of A up to 4096^3, else a bounded row
sample). Warm-up runs at least --warmup steps and at least 100 ms, which puts
the timed region past the clock transient that follows a cold start (the
first GEMMs after idle run up to 1.4x slower for about 25 ms), whatever
--warmup says.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
                       [--mode fast|accurate] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0      # MI355X dense INT8 MFMA (no sparsity)
FP64_PEAK_TFLOPS = 78.6      # MI355X FP64 matrix peak
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # MI355X settles its clock for this load within ~25 ms of a cold start
    # (the first GEMMs after idle swing between 0.85 and 1.2 ms); 40 warm-up
    # steps (~50 ms) put the timed region in the sustained state
    p.add_argument("--steps", type=int, default=40)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--config", default="spread1.0_4096_n16")
    p.add_argument("--mode", default="fast", choices=["fast", "accurate", "original"],
                   help="original: the comparison stand-in for the original fast-mode rule")
    p.add_argument("--num-moduli", type=int, default=0, help="override the workload's number of moduli")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip the accurate-mode and native-FP64 context runs")
    p.add_argument("--cpu-rows", type=int, default=0, help="rows of A in the oracle sample (0: automatic)")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB (3 times) for HBM counter calibration")
    return p.parse_args()


def gemm_source_hash():
    """SHA-256 of the GEMM's source with comments and blank lines removed: the
    GEMM section of kernels.hip, its launcher (tile shape and kernel choice,
    grid), and the tiling constants and ModConsts / Layout structs of common.h.
    It changes when that code does, not when only comments or other kernels do."""
    import hashlib
    import re

    def code(src):
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        lines = [re.sub(r"//.*$", "", line).rstrip() for line in src.splitlines()]
        return "\n".join(line for line in lines if line.strip())

    src = open(os.path.join(ROOT, "rns_emulated_fp64_amd", "csrc", "kernels.hip")).read()
    sec = src[src.index("// Step 3: INT8 GEMM"):src.index("// Steps 4 + 5")]
    launch = src[src.index("static int compute_units()"):src.index("hipError_t launch_gemm_raw(")]
    common = open(os.path.join(ROOT, "rns_emulated_fp64_amd", "csrc", "common.h")).read()
    parts = re.findall(r"constexpr int k(?:TileM|TileN|KPad) = \d+;", common)
    parts += re.findall(r"struct (?:ModConsts|Layout) \{.*?\};", common, flags=re.S)
    return hashlib.sha256("\n".join(code(x) for x in [sec, launch] + parts).encode()).hexdigest()


def gemm_kernel_name():
    """The INT8 GEMM kernel the headline workload runs on (256 x 256 tiles, more
    tiles than compute units, more than four 64-deep stages): the persistent one
    unless OZ2_GEMM_KERNEL=blocks."""
    return "k_gemm<EPI_MOD>" if os.environ.get("OZ2_GEMM_KERNEL") == "blocks" else "k_gemm_persistent"


def gemm_traffic_bytes():
    """HBM bytes per GEMM launch from the committed counter runs, or None.

    The figure is used only while the GEMM's code still hashes to the one the
    counters were taken on.
    """
    stem = "k_gemm" if gemm_kernel_name() == "k_gemm<EPI_MOD>" else gemm_kernel_name()
    path = os.path.join(ROOT, "profiles", f"{stem}_spread1.0_4096_n16_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if gemm_source_hash() != rec["gemm_code_sha256"]:
        return None
    return float(rec["traffic_bytes_per_launch"])


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_info():
    """CPU model and core counts of the host this runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        usable = os.cpu_count()
    return dict(cpu_model=model, nproc=usable, cpu_count=os.cpu_count())


def _sclk_files():
    """sysfs files listing the GPU core clock levels (the current one starred)."""
    import glob
    return sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))


def _read_sclk(path):
    """Current core clock in MHz from a pp_dpm_sclk listing, or None."""
    try:
        with open(path) as fh:
            for line in fh:
                if "*" in line:
                    tok = line.split(":", 1)[1].strip().split()[0].lower()
                    return int(float(tok.replace("mhz", "")))
    except (OSError, ValueError, IndexError):
        return None
    return None


def sample_clocks(step, torch, samples=40, every_steps=4):
    """Core clock readings (MHz) from sysfs while the product runs in a loop,
    after the timed region so the timed steps are untouched; reported as
    min / median / max of the samples, or None where sysfs has no listing."""
    files = _sclk_files()
    if not files:
        return None
    vals = []
    for _ in range(samples):
        for _ in range(every_steps):
            step()
        v = _read_sclk(files[0])
        if v is not None:
            vals.append(v)
    torch.cuda.synchronize()
    if not vals:
        return None
    vals.sort()
    return dict(source=files[0].replace("/sys/class/drm/", ""), samples=len(vals), min_mhz=vals[0],
                median_mhz=vals[len(vals) // 2], max_mhz=vals[-1])


def phase_bytes(m, n, k, N, elem, cplx):
    """Algorithmic HBM bytes of each phase: operands read, residue planes
    written and read once (int8), C written; no padding, no re-reads."""
    planes = 3 * N if cplx else N
    ops = elem * (m * k + k * n)
    res = planes * (m * k + n * k)
    prod = planes * m * n
    return dict(scale=ops, split=ops + res, gemm=res + prod, crt=prod + elem * m * n)


def time_steps(fn, steps, warmup, torch, settle_ms=60.0):
    """Mean ms per call of fn over `steps` calls, after at least `warmup`
    calls and at least `settle_ms` of warm-up (the clock settles under load)."""
    t0 = time.perf_counter()
    done = 0
    while done < warmup or (time.perf_counter() - t0) * 1e3 < settle_ms:
        fn()
        torch.cuda.synchronize()
        done += 1
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def cpu_baseline_leg(A, B, C_gpu, N, mode, rows_wanted, gpu_e=None, gpu_f=None):
    """The oracle (as it stands) on the first rows of A times all of B: every
    row up to 4096^3 work, else a bounded sample of about that size."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    omp_threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    m, k = A.shape
    n = B.shape[1]
    rows = rows_wanted or max(8, min(m, int(4096 * (4096 / max(k, 1)) * (4096 / max(n, 1)))))
    rows = min(rows, m)
    single = A.dtype == np.float32
    emul = O.os2_sgemm if single else O.os2_dgemm
    log(f"cpu_baseline: oracle on {rows} rows x {n} columns, k={k}, N={N}, {mode}")
    t0 = time.perf_counter()
    r = emul(A[:rows], B, N, mode)
    t = time.perf_counter() - t0
    value = 2.0 * rows * n * k / t / 1e12
    Cs = C_gpu[:rows]
    bits = np.uint32 if single else np.uint64
    diff = (Cs.view(bits) != r["C"].view(bits)) & ~(np.isnan(Cs) & np.isnan(r["C"]))
    er = min(rows, 128)  # accuracy against the double-double reference on the first rows
    A64, B64 = A[:er].astype(np.float64), B.astype(np.float64)
    hi, lo = O.dd_gemm(A64, B64)
    err = O.error_metrics(Cs[:er].astype(np.float64), hi, lo, A64, B64)
    native = O.error_metrics((A[:er] @ B).astype(np.float64), hi, lo, A64, B64)
    nat = "fp32" if single else "fp64"
    # the host's native product (numpy / OpenBLAS) on the same sample and cores, as context
    t0 = time.perf_counter()
    _ = A[:rows] @ B
    t_host = time.perf_counter() - t0
    # exponents: GPU against the oracle on the same rows and all columns
    # (a mismatch is allowed only at a rounding boundary; expected 0)
    exp_mm = None
    if gpu_e is not None and gpu_f is not None:
        as_int = lambda v: [(-(2 ** 31) if x is None else int(x)) for x in v]
        exp_mm = int(sum(a != b for a, b in zip(as_int(r["e"]), gpu_e[:rows]))) + \
            int(sum(a != b for a, b in zip(as_int(r["f"]), gpu_f)))
    hi_ = host_info()
    return dict(value=value, unit="TFLOPS", cores=max(omp_threads, blas_threads), kind="oracle",
                sample=(f"all {rows} rows of A times all of B" if rows == m else
                        f"rows 0..{rows - 1} of A times all of B") + f" ({rows}x{n}x{k}, N={N}, {mode}); "
                       f"{t:.2f} s; OpenMP {omp_threads} threads, BLAS {blas_threads} threads",
                **hi_), \
        dict(parity_mismatches=int(diff.sum()), parity_entries=int(Cs.size), exponent_mismatches=exp_mm,
             exponents_compared=(rows + n) if exp_mm is not None else 0, error_rows=er, **err,
             **{f"native_{nat}_E_cw": native["E_cw"], f"native_{nat}_E_el": native["E_el"],
                f"host_native_{nat}_gemm_tflops": round(2.0 * rows * n * k / t_host / 1e12, 4)})


def cpu_baseline_complex(A, B, C_gpu, N, rows_wanted):
    """The oracle's complex emulation on the first rows of A times all of B."""
    import numpy as np
    import oracle as O
    m, k = A.shape
    n = B.shape[1]
    rows = min(m, rows_wanted or max(8, int(1024 * (4096 / max(k, 1)) * (4096 / max(n, 1)))))
    log(f"cpu_baseline: complex oracle on {rows} rows x {n} columns, k={k}, N={N}")
    t0 = time.perf_counter()
    r = O.os2_zgemm(A[:rows], B, N)
    t = time.perf_counter() - t0
    Cs = C_gpu[:rows]
    same = lambda x, y: (x.view(np.uint64) == y.view(np.uint64)) | (np.isnan(x) & np.isnan(y))
    ok = same(np.ascontiguousarray(Cs.real), np.ascontiguousarray(r["C"].real)) & \
        same(np.ascontiguousarray(Cs.imag), np.ascontiguousarray(r["C"].imag))
    return dict(value=8.0 * rows * n * k / t / 1e12, unit="TFLOPS", cores=int(os.environ.get("OMP_NUM_THREADS",
                os.cpu_count() or 1)), kind="oracle",
                sample=f"rows 0..{rows - 1} of A times all of B ({rows}x{n}x{k} complex, N={N}); {t:.2f} s"), \
        dict(parity_mismatches=int((~ok).sum()), parity_entries=int(Cs.size))


def sweep_main(args, cfg, torch, oz, W, np):
    """The scale sweep ([G] Problemstellung / Methodik 2): A = 2^s ones and
    2^s U(-1,1), proposed fast mode vs the stand-in for the original rule.
    Accuracy E_cw on sampled rows against the double-double reference, and CRT
    success on sampled entries against the exact integers for the exponents
    each mode chose. One JSON line."""
    import oracle as O
    m = n = k = cfg["m"]
    N = cfg["num_moduli"]
    ones, ua, B = W.scale_sweep_case(m, cfg["seed"])
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    dB = torch.from_numpy(np.ascontiguousarray(B.T)).to(dev)
    dC = torch.empty((n, m), dtype=torch.float64, device=dev)
    wb = oz.ozaki2_workspace_size(m, n, k, N, oz.FAST)
    ws = torch.empty(wb, dtype=torch.uint8, device=dev)
    e_dev = torch.empty(m, dtype=torch.int32, device=dev)
    f_dev = torch.empty(n, dtype=torch.int32, device=dev)
    dbg_wb = oz.ozaki2_debug_workspace_size(m, n, k, N, oz.FAST)
    dbg_ws = torch.empty(dbg_wb, dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(m, 16, replace=False)).tolist()
    cols = np.sort(rng.choice(n, 16, replace=False)).tolist()
    out = []
    for name, A0 in (("ones", ones), ("U(-1,1)", ua)):
        hi, lo = O.dd_gemm(A0[rows], B)
        for s in (-64, -32, 0, 32, 64):
            As = np.ldexp(A0, s)
            dA = torch.from_numpy(np.ascontiguousarray(As.T)).to(dev)
            for mode in ("fast", "original"):
                md = oz.MODES[mode]

                def step():
                    st = oz.ozaki2_dgemm_ws(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, dC.data_ptr(), m, N, md,
                                            ws.data_ptr(), wb, stream)
                    if st:
                        raise RuntimeError(oz.status_string(st))

                ms = time_steps(step, max(args.steps // 4, 3), 1, torch)
                st = oz.ozaki2_dgemm_debug(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, dC.data_ptr(), m, N, md,
                                           dbg_ws.data_ptr(), dbg_wb, e_dev.data_ptr(), f_dev.data_ptr(), None, None,
                                           None, None, stream)
                assert st == 0
                torch.cuda.synchronize()
                C = dC.cpu().numpy().T
                e = e_dev.cpu().numpy().tolist()
                f = f_dev.cpu().numpy().tolist()
                err = O.error_metrics(np.ldexp(C[rows], -s), hi, lo, A0[rows], B)
                try:
                    er, fc = [e[i] for i in rows], [f[j] for j in cols]
                    Y = O.scaled_integers(As[rows], er).dot(O.scaled_integers(B[:, cols].T, fc).T)
                    crt_ok = bool(np.array_equal(C[np.ix_(rows, cols)], O.unscale(Y, er, fc)))
                except OverflowError:
                    crt_ok = False
                out.append(dict(matrix=name, s=s, mode="proposed" if mode == "fast" else "original stand-in",
                                E_cw=float(err["E_cw"]), crt_ok_on_sample=crt_ok, ms=round(ms, 4),
                                e_row0=int(e[0])))
                log(f"{name} 2^{s} {mode}: E_cw {err['E_cw']:.3e}, crt_ok {crt_ok}, {ms:.3f} ms")
            del dA
    worst = max(r["E_cw"] for r in out if r["mode"] == "proposed")
    line = dict(metric="scale sweep at 2048^3, N=14: max E_cw over alpha = 2^s (proposed fast mode)",
                value=worst, unit="E_cw", n_gpus=1, steps=max(args.steps // 4, 3), warmup=1,
                higher_is_better=False, scaling="weak", vs_baseline=None, dtype="int8", data="synthetic",
                config=dict(workload=args.config, m=m, n=n, k=k, num_moduli=N, s=[-64, -32, 0, 32, 64],
                            sample_rows=len(rows), sample_cols=len(cols)),
                sweep=out)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the product would "
              "shard by output tiles, with no exchange in fast mode).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy_mib:
        # a plain copy kernel of known size: reads and writes exactly this many bytes
        nbytes = args.calibrate_copy_mib << 20
        src = torch.ones(nbytes // 8, dtype=torch.float64, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(calibration="copy", bytes_read=nbytes, bytes_written=nbytes, launches=3)))
        return

    import rns_emulated_fp64_amd as oz
    import workloads as W

    # a dedicated stream (default priority), current for the whole run: the
    # library calls, their timing events and the comparators all run on it
    torch.cuda.set_stream(torch.cuda.Stream(device=torch.device("cuda:0")))
    cfg = W.CONFIGS[args.config]
    if cfg["kind"] == "sweep":
        return sweep_main(args, cfg, torch, oz, W, np)
    m, n, k, N = cfg["m"], cfg["n"], cfg["k"], cfg["num_moduli"]
    N = args.num_moduli or N
    single = bool(cfg.get("single"))
    cplx = bool(cfg.get("complex"))
    md = oz.MODES[args.mode]
    log(f"generating {args.config} ({m}x{k} @ {k}x{n}), N={N}, mode={args.mode}")
    A, B = W.make(args.config)
    dev = torch.device("cuda:0")
    dA = torch.from_numpy(np.ascontiguousarray(A.T)).to(dev)  # column-major A, lda = m
    dB = torch.from_numpy(np.ascontiguousarray(B.T)).to(dev)  # column-major B, ldb = k
    dC = torch.empty((n, m), dtype=torch.complex128 if cplx else torch.float32 if single else torch.float64,
                     device=dev)
    gemm_ws = oz.ozaki2_zgemm_ws if cplx else oz.ozaki2_sgemm_ws if single else oz.ozaki2_dgemm_ws
    stream = torch.cuda.current_stream(dev).cuda_stream

    def workspace(mode_id):
        wb = oz.ozaki2_zgemm_workspace_size(m, n, k, N) if cplx else oz.ozaki2_workspace_size(m, n, k, N, mode_id)
        return torch.empty(wb, dtype=torch.uint8, device=dev), wb

    ws, wbytes = workspace(md)

    def step(mode_id=md, w=None, wb=None):
        w = ws if w is None else w
        wb = wbytes if wb is None else wb
        st = gemm_ws(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, dC.data_ptr(), m, N, mode_id, w.data_ptr(), wb,
                     stream)
        if st:
            raise RuntimeError(oz.status_string(st))

    # warm-up: at least --warmup steps and at least 100 ms of steps, so the
    # timed region starts after the clock transient of a cold start
    settle_ms = 100.0
    t0 = time.perf_counter()
    warm = 0
    while warm < args.warmup or (time.perf_counter() - t0) * 1e3 < settle_ms:
        step()
        warm += 1
        if warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warmup_ms = (time.perf_counter() - t0) * 1e3
    # timed region: HIP events attached to the GEMM launch of every step (same stream)
    oz.ozaki2_timing_enable(args.steps, all_phases=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    per_call = sorted(c["gemm"] for c in oz.ozaki2_timing_read_calls(args.steps))
    gemm_avg = sum(per_call) / max(len(per_call), 1)
    gemm_min = per_call[0] if per_call else 0.0
    gemm_med = per_call[len(per_call) // 2] if per_call else 0.0
    # per-phase breakdown from a separate, untimed pass
    nb = max(3, min(args.steps, 10))
    oz.ozaki2_timing_enable(nb, all_phases=True)
    for _ in range(nb):
        step()
    phase_ms, pcalls = oz.ozaki2_timing_read()
    oz.ozaki2_timing_enable(0)
    phase_avg = {p: v / max(pcalls, 1) for p, v in phase_ms.items()}
    log(f"{ms:.3f} ms/step; GEMM {gemm_avg:.4f} ms (timed region); phases {phase_avg}")
    elem = (16 if not single else 8) if cplx else (4 if single else 8)
    pbytes = phase_bytes(m, n, k, N, elem, cplx)
    phase_gbs = {p: round(pbytes[p] / (phase_avg[p] * 1e-3) / 1e9, 1) for p in pbytes if phase_avg.get(p, 0) > 0}
    clocks = None if args.no_extras else sample_clocks(step, torch)

    flops = (8.0 if cplx else 2.0) * m * n * k  # a complex multiply-add is 8 real flops
    tflops = flops / (ms * 1e-3) / 1e12
    # one INT8 GEMM per modulus (three for complex products), all in one launch
    int8_ops = N * (3 if cplx else 1) * 2.0 * m * n * k
    gemm_tops = int8_ops / (gemm_avg * 1e-3) / 1e12
    traffic = gemm_traffic_bytes() if args.config == "spread1.0_4096_n16" and args.mode == "fast" else None
    roofline = dict(bound="mfma", achieved=round(gemm_tops, 2), peak=INT8_PEAK_TOPS, unit="TFLOP/s",
                    frac=round(gemm_tops / INT8_PEAK_TOPS, 4), traffic=traffic,
                    kernel=gemm_kernel_name(), ops_per_launch=int8_ops, dtype="int8")

    C = dC.cpu().numpy().T  # C of the last step
    extras = {}
    if cplx and not args.no_extras:
        Azt = torch.from_numpy(A).to(dev)
        Bzt = torch.from_numpy(B).to(dev)
        ms8 = time_steps(lambda: torch.mm(Azt, Bzt), max(args.steps // 2, 3), 2, torch)
        extras["native_complex128_gemm_tflops"] = round(flops / (ms8 * 1e-3) / 1e12, 3)
        del Azt, Bzt
    elif not args.no_extras:
        # accurate mode (the other mode) and native FP64 on the same operands, as context
        other = "accurate" if args.mode != "accurate" else "fast"
        w2, wb2 = workspace(oz.MODES[other])
        ms2 = time_steps(lambda: step(oz.MODES[other], w2, wb2), max(args.steps // 2, 3), 2, torch)
        extras[f"{other}_mode_tflops"] = round(flops / (ms2 * 1e-3) / 1e12, 3)
        extras[f"{other}_mode_ms_per_step"] = round(ms2, 4)
        del w2
        step()  # restore C of the benchmarked mode
        torch.cuda.synchronize()
        At = torch.from_numpy(A).to(dev)
        Bt = torch.from_numpy(B).to(dev)
        ms3 = time_steps(lambda: torch.mm(At, Bt), max(args.steps // 2, 3), 2, torch)
        extras[f"native_fp{32 if single else 64}_gemm_tflops"] = round(flops / (ms3 * 1e-3) / 1e12, 3)
        del At, Bt
        if not single:
            # the single-precision emulation ([G] Zentrale Beiträge) on its 4096^3 workload, as context
            As, Bs = W.make("sgemm_spread1.0_4096_n8")
            cs = W.CONFIGS["sgemm_spread1.0_4096_n8"]
            ms_, ns_, ks_, Ns = cs["m"], cs["n"], cs["k"], cs["num_moduli"]
            dAs = torch.from_numpy(np.ascontiguousarray(As.T)).to(dev)
            dBs = torch.from_numpy(np.ascontiguousarray(Bs.T)).to(dev)
            dCs = torch.empty((ns_, ms_), dtype=torch.float32, device=dev)
            wbs = oz.ozaki2_workspace_size(ms_, ns_, ks_, Ns, oz.FAST)
            wss = torch.empty(wbs, dtype=torch.uint8, device=dev)

            def sstep():
                st = oz.ozaki2_sgemm_ws(ms_, ns_, ks_, dAs.data_ptr(), ms_, dBs.data_ptr(), ks_, dCs.data_ptr(), ms_,
                                        Ns, oz.FAST, wss.data_ptr(), wbs, stream)
                if st:
                    raise RuntimeError(oz.status_string(st))

            ms5 = time_steps(sstep, max(args.steps, 5), 3, torch)
            sflops = 2.0 * ms_ * ns_ * ks_
            extras["sgemm_n8_tflops"] = round(sflops / (ms5 * 1e-3) / 1e12, 3)
            extras["sgemm_n8_ms_per_step"] = round(ms5, 4)
            Ats = torch.from_numpy(As).to(dev)
            Bts = torch.from_numpy(Bs).to(dev)
            ms6 = time_steps(lambda: torch.mm(Ats, Bts), max(args.steps // 2, 3), 2, torch)
            extras["native_fp32_gemm_tflops"] = round(sflops / (ms6 * 1e-3) / 1e12, 3)
            del dAs, dBs, dCs, wss, Ats, Bts
            # complex products (ZGEMM, Gauss' three products per modulus) on complex
            # operands of the same spread at the same size; 8mnk real flops
            Az, Bz = W.make("zgemm_spread1.0_4096_n16")
            dAz = torch.from_numpy(np.ascontiguousarray(Az.T)).to(dev)  # column-major, interleaved
            dBz = torch.from_numpy(np.ascontiguousarray(Bz.T)).to(dev)
            dCz = torch.empty((n, m), dtype=torch.complex128, device=dev)
            wbz = oz.ozaki2_zgemm_workspace_size(m, n, k, N)
            wsz = torch.empty(wbz, dtype=torch.uint8, device=dev)

            def zstep():
                st = oz.ozaki2_zgemm_ws(m, n, k, dAz.data_ptr(), m, dBz.data_ptr(), k, dCz.data_ptr(), m, N, oz.FAST,
                                        wsz.data_ptr(), wbz, stream)
                if st:
                    raise RuntimeError(oz.status_string(st))

            ms7 = time_steps(zstep, max(args.steps // 2, 3), 2, torch)
            extras[f"zgemm_n{N}_tflops"] = round(4 * flops / (ms7 * 1e-3) / 1e12, 3)
            extras[f"zgemm_n{N}_ms_per_step"] = round(ms7, 4)
            del wsz, dCz
            Azt = torch.from_numpy(Az).to(dev)
            Bzt = torch.from_numpy(Bz).to(dev)
            ms8 = time_steps(lambda: torch.mm(Azt, Bzt), max(args.steps // 2, 3), 2, torch)
            extras["native_complex128_gemm_tflops"] = round(4 * flops / (ms8 * 1e-3) / 1e12, 3)
            del dAz, dBz, Azt, Bzt
        # the vendor INT8 GEMM (torch._int_mm = hipBLASLt) on random int8 of one
        # modulus' shape, as context for the INT8 roofline fraction
        try:
            Ai = torch.randint(-128, 128, (m, k), dtype=torch.int8, device=dev)
            Bi = torch.randint(-128, 128, (n, k), dtype=torch.int8, device=dev).t()  # column-major k x n
            ms4 = time_steps(lambda: torch._int_mm(Ai, Bi), max(args.steps, 5), 3, torch)
            extras["vendor_int8_gemm_tops"] = round(2.0 * m * n * k / (ms4 * 1e-3) / 1e12, 1)
            del Ai, Bi
        except Exception as ex:  # pragma: no cover - context only
            log(f"vendor int8 GEMM not measured: {ex}")

    cpu = None
    accuracy = None
    if not args.no_cpu_baseline and not cplx:
        # the GPU's exponents of this product (debug entry point, e and f only)
        dbg_wb = oz.ozaki2_debug_workspace_size(m, n, k, N, md)
        dbg_ws = torch.empty(dbg_wb, dtype=torch.uint8, device=dev)
        e_dev = torch.empty(max(m, 1), dtype=torch.int32, device=dev)
        f_dev = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
        dbg = oz.ozaki2_sgemm_debug if single else oz.ozaki2_dgemm_debug
        st = dbg(m, n, k, dA.data_ptr(), m, dB.data_ptr(), k, dC.data_ptr(), m, N, md, dbg_ws.data_ptr(), dbg_wb,
                 e_dev.data_ptr(), f_dev.data_ptr(), None, None, None, None, stream)
        if st:
            raise RuntimeError(oz.status_string(st))
        torch.cuda.synchronize()
        gpu_e, gpu_f = e_dev[:m].cpu().tolist(), f_dev[:n].cpu().tolist()
        del dbg_ws
        cpu, accuracy = cpu_baseline_leg(A, B, C, N, args.mode, args.cpu_rows, gpu_e, gpu_f)
    elif not args.no_cpu_baseline:
        cpu, accuracy = cpu_baseline_complex(A, B, C, N, args.cpu_rows)

    line = dict(
        metric=("emulated complex FP64 TFLOPS (8mnk/t)" if cplx else "emulated FP32 TFLOPS (2mnk/t)" if single else
                "emulated FP64 TFLOPS (2mnk/t) at 4096^3, % INT8 MFMA peak; max rel err"),
        value=round(tflops, 3), unit="TFLOPS", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms, 4), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="int8", data="synthetic",
        config=dict(workload=args.config, m=m, n=n, k=k, num_moduli=N, mode=args.mode,
                    entries=("(U(0,1)-0.5)*exp(%s*N(0,1))" % cfg.get("phi")) if cfg["kind"] == "spread"
                    else "U(-1,1)", seed=cfg["seed"]),
        emulated_vs_fp64_peak=round(tflops / FP64_PEAK_TFLOPS, 3),
        gemm_int8_peak_frac=roofline["frac"],
        gemm_ms_timed_region=round(gemm_avg, 4),
        gemm_ms_timed_min=round(gemm_min, 4),
        gemm_ms_timed_median=round(gemm_med, 4),
        warmup_steps_run=warm,
        warmup_ms=round(warmup_ms, 1),
        phase_ms={p: round(v, 4) for p, v in phase_avg.items()},
        phase_gbs=phase_gbs,
        phase_bytes=pbytes,
        gpu_clocks=clocks,
        roofline=roofline,
        cpu_baseline=cpu,
        accuracy=accuracy,
        **extras,
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
