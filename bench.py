"""Benchmark: GEMM TFLOPS of pgemm on one MI355X, with roofline and CPU baseline.

One step = one call C <- alpha*A*B + beta*C through the C ABI on inputs that
are already resident in HBM: gemm_f32 / gemm_f64, or gemm_*_ws with the
workspace the library asks for when the tiles of C leave a partly filled last
round, or matmat_f64 for the row-major fp64 workload.  W untimed warmup
steps (continued for at least --min-warmup-seconds), then exactly K timed
steps back to back, bracketed by torch.cuda.synchronize() and, on the launch
stream, by two HIP events.

Prints ONE JSON line.  ``value`` is the whole-job throughput in TFLOPS
(2*M*N*K per step / wall time per step).  ``roofline`` compares the
throughput the two events measure (the stream's GPU time for the K steps)
with MI355X's dense fp32 (or fp64) matrix peak.  ``secondary`` holds one such
line for every other configuration point (steps scaled up for short kernels:
about 50 ms of GPU time each).  ``cpu_baseline`` times the CPU oracle (test
infrastructure, built from oracle/oracle.c) on a bounded sample of the
primary workload: the first J columns of C, with J chosen for roughly 10-20 s
of CPU work; the same sample also checks the GPU's first output against the
oracle.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--secondary NAME ...] [--sweep]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gemm_inputs as gi  # noqa: E402

PEAK_TFLOPS = {"f32": 157.3, "f64": 78.6}  # MI355X dense matrix peaks
HBM_PEAK_GBS = 8000.0
METRIC = "GEMM TFLOPS (fp32, M=N=K=2048/8192) and % of MI355X fp32 matrix peak"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sgemm_sweep_8192")
    ap.add_argument("--secondary", nargs="*",
                    default=["sgemm_2048", "sgemm_128", "sgemm_sweep_512", "sgemm_sweep_1024",
                             "sgemm_sweep_2048", "sgemm_sweep_4096", "sgemm_ragged",
                             "dgemm_rowmajor", "sgemm_shard_8192_g8"],
                    help="workloads timed after the primary one, each on its own line "
                         "(default: every configuration point)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--min-warmup-seconds", type=float, default=0.3,
                    help="keep warming up (untimed) until this much wall time has passed")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the JSON line: every workload once, GPU time, parity "
                         "against the oracle and the oracle's own time, as a markdown table")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run two device-to-device copies of this many MiB (a plain "
                         "copy of known size, to scale HBM byte counters)")
    return ap.parse_args()


class Resident:
    """A workload's operands on the GPU, plus a launcher bound to them."""

    def __init__(self, name):
        import torch
        import precision_gemm_02_amd as pg
        self.name = name
        self.p = p = gi.workload(name)
        self.dt = "f32" if p.dtype == np.float32 else "f64"
        self.A = torch.from_numpy(p.A).cuda()
        self.B = torch.from_numpy(p.B).cuda()
        self.C0 = torch.from_numpy(p.C).cuda()
        self.C = self.C0.clone()
        self.pg = pg
        if p.rowmajor:   # lecture form: C^T = B^T A^T, column-major (n x m)
            self.args = (p.n, p.m, p.k, p.alpha, self.B.data_ptr(), p.ldb, self.A.data_ptr(),
                         p.lda, p.beta, self.C.data_ptr(), p.ldc)
        else:
            self.args = (p.m, p.n, p.k, p.alpha, self.A.data_ptr(), p.lda, self.B.data_ptr(),
                         p.ldb, p.beta, self.C.data_ptr(), p.ldc)
        self.flops = 2.0 * p.m * p.n * p.k
        self.stream = torch.cuda.current_stream()
        # The K iterations of a partly filled last round of tiles are shared
        # by stream-K workgroups when the library is given the workspace it
        # asks for (gemm_*_ws); shapes that fill whole rounds ask for none
        # and use the plain entry point.
        self.ws_bytes = 0
        self.ws = None
        if not p.rowmajor:
            wsfn = pg.workspace_f32 if self.dt == "f32" else pg.workspace_f64
            self.ws_bytes = int(wsfn(*self.args[:3]))
            if self.ws_bytes > 0:
                self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        if p.rowmajor:
            self.entry = "matmat_f64"
        else:
            self.entry = ("gemm_%s_ws" if self.ws_bytes else "gemm_%s") % self.dt
        # the kernel the entry point launches, and how many stream-K
        # workgroups share the last round (0: none, no fix-up kernel)
        sel = pg.select_ws_f32 if self.dt == "f32" else pg.select_ws_f64
        vid, self.sk_wgs, self.strip_rows = sel(*self.args, self.ws_bytes)
        self.variant = pg.variants().get(vid, "none")

        # One C-ABI call per step, its arguments converted once here: the
        # launch loop of a microsecond kernel must not be paced by Python.
        lib, sh = pg.library(), self.stream.cuda_stream
        if p.rowmajor:
            fn = lib.matmat_f64
            cargs = (p.lda, p.ldb, p.ldc, self.A.data_ptr(), self.B.data_ptr(),
                     self.C.data_ptr(), p.m, p.k, p.n, sh)
        elif self.ws_bytes:
            fn = lib.gemm_f32_ws if self.dt == "f32" else lib.gemm_f64_ws
            cargs = (*self.args, self.ws.data_ptr(), self.ws_bytes, sh)
        else:
            fn = lib.gemm_f32 if self.dt == "f32" else lib.gemm_f64
            cargs = (*self.args, sh)
        self._fn, self._cargs = fn, cargs

    def launch(self):
        st = self._fn(*self._cargs)
        if st != 0:
            raise RuntimeError("%s: status %d (%s)" % (self.entry, st,
                                                      self.pg.status_string(st)))

    def reset_c(self):
        if self.p.beta != 0:
            self.C.copy_(self.C0)

    def algorithmic_bytes(self):
        p = self.p
        s = 4 if self.dt == "f32" else 8
        return s * (p.m * p.k + p.k * p.n + p.m * p.n * (1 + (p.beta != 0)))


def warm_up(r: Resident, warmup: int, min_warm_s: float):
    """At least ``warmup`` launches, continued until ``min_warm_s`` of wall time
    has passed (the GPU raises its clock over a few hundred ms of sustained
    load; a short kernel timed right after an idle gap measures the ramp, not
    the kernel).  C is restored every 64 launches (|beta| > 1 grows it).
    Returns (launches, wall seconds per launch over the last batch)."""
    import torch
    n_warm = 0
    t_end = time.perf_counter() + min_warm_s
    t_batch, n_batch = time.perf_counter(), 0
    per = None
    while n_warm < warmup or time.perf_counter() < t_end:
        r.launch()
        n_warm += 1
        n_batch += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()
            now = time.perf_counter()
            per = (now - t_batch) / n_batch
            t_batch, n_batch = now, 0
        if n_warm % 64 == 0:
            r.reset_c()
    torch.cuda.synchronize()
    if per is None:
        per = (time.perf_counter() - t_batch) / max(n_batch, 1)
    r.reset_c()
    torch.cuda.synchronize()
    return n_warm, per


def timed_steps(r: Resident, steps: int):
    """The timed region: exactly ``steps`` launches back to back between two
    synchronizations, with a HIP event recorded on the launch stream right
    before the first launch and right after the last.  Returns (wall ms per
    step, GPU ms per step from the two events).  The events see the stream's
    own time for the steps (every kernel a step launches, and the gaps
    between launches), not the host's."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(r.stream)
    for _ in range(steps):
        r.launch()
    e1.record(r.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    r.reset_c()
    torch.cuda.synchronize()
    return wall / steps * 1e3, gpu_ms / steps


def auto_steps(r: Resident, base: int, per_launch_s: float, region_s: float = 0.05) -> int:
    """Steps for a secondary workload: at least ``base``, and enough for about
    ``region_s`` of GPU time (microsecond kernels need thousands of steps for
    a stable average), at most 20000; at most 300 when |beta| > 1, so that C
    stays finite."""
    n = max(base, int(region_s / max(per_launch_s, 1e-7)))
    n = min(n, 20000)
    if abs(r.p.beta) > 1:
        n = min(n, 300)
    return n


PROFILES = os.path.join(ROOT, "profiles")
LIB = os.path.join(ROOT, "precision_gemm_02_amd", "libpgemm.so")


def _build_module():
    """precision_gemm_02_amd/build.py, loaded by path (no library import)."""
    import importlib.util
    path = os.path.join(ROOT, "precision_gemm_02_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_pgemm_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def library_digest() -> str:
    """Digest of the kernel sources and build flags (build.source_digest):
    the same at any build path, so counters recorded from one build apply to
    another build of the same sources.  "stale" if libpgemm.so is older than
    a source file (the sources no longer describe the library that runs)."""
    if not os.path.exists(LIB):
        return "unbuilt"
    b = _build_module()
    newest = max(os.path.getmtime(os.path.join(b.CSRC, f)) for f in os.listdir(b.CSRC))
    newest = max(newest, os.path.getmtime(os.path.join(b.INCLUDE, "pgemm.h")))
    if os.path.getmtime(LIB) + 1.0 < newest:
        return "stale"
    return b.source_digest()


_warned = set()


def recorded_profile(variant: str, workload: str) -> dict:
    """Values measured by rocprofv3 counter runs for this variant and
    workload, as recorded in profiles/*counters*.md, or {} if none matches
    them and the current sources (the kernel changed since they were
    taken); a warning names what did not match."""
    if not os.path.isdir(PROFILES):
        return {}
    digest = library_digest()
    seen = []
    for f in sorted(os.listdir(PROFILES)):
        if "counters" not in f:
            continue
        kv = {}
        for line in open(os.path.join(PROFILES, f)):
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                kv[k.strip("`")] = v.strip().strip("`")
        if kv.get("variant") == variant and kv.get("workload") == workload:
            if kv.get("library_digest") == digest:
                return kv
            seen.append((f, kv.get("library_digest")))
    if (variant, workload) not in _warned:
        _warned.add((variant, workload))
        log("no recorded counters for %s on %s with source digest %s%s" % (
            variant, workload, digest,
            "" if not seen else " (recorded with other digests: %s)" % ", ".join(
                "%s in %s" % (d, f) for f, d in seen)))
    return {}


def recorded_traffic(variant: str, workload: str):
    """HBM bytes per launch from the recorded counters, or None."""
    kv = recorded_profile(variant, workload)
    return float(kv["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in kv else None


def recorded_counters(variant: str, workload: str):
    """MFMA-busy share and LDS bank-conflict cycles from the recorded
    counters (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE and
    SQ_LDS_BANK_CONFLICT, per launch), or None."""
    kv = recorded_profile(variant, workload)
    if "mfma_util" not in kv or "lds_bank_conflict_cycles" not in kv:
        return None
    return {"mfma_util": float(kv["mfma_util"]),
            "lds_bank_conflict_cycles": float(kv["lds_bank_conflict_cycles"]),
            "source": "rocprofv3 --pmc, profiles/ (same kernel sources and build flags)"}


def device_peak(dt: str):
    """(matrix peak in TFLOP/s from the device's own compute-unit count and
    peak clock, CUs, clock MHz): 256 flop per CU per cycle for fp32, 128 for
    fp64 (the published peaks are these at 256 CUs and 2.4 GHz)."""
    import precision_gemm_02_amd as pg
    cus, khz = pg.device_info()
    per_cycle = 256 if dt == "f32" else 128
    return cus * khz * 1e3 * per_cycle / 1e12, cus, khz / 1e3


def roofline(r: Resident, gpu_ms: float):
    """Matrix-core roofline of the step: algorithmic flops per step (2MNK)
    over the GPU time per step that two HIP events around the timed region
    measured on the launch stream.  A step is one library call: the GEMM
    kernel plus, where the shape needs them, the strip kernel or the
    stream-K fix-up kernel, which this time includes.  `peak` is the
    published one; the peak recomputed from the device's properties is given
    beside it.  The largest problems are bound by the matrix cores; the
    smallest (128^3) by launch latency, and its time is also given in us."""
    achieved = r.flops / (gpu_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[r.dt]
    dpeak, cus, mhz = device_peak(r.dt)
    return {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "peak_device_props": round(dpeak, 2), "frac_device_props": round(achieved / dpeak, 4),
            "device": {"cus": cus, "clock_mhz": mhz},
            "traffic": recorded_traffic(r.variant, r.name),
            "counters": recorded_counters(r.variant, r.name),
            "algorithmic_bytes": r.algorithmic_bytes(),
            "kernel": r.variant, "stream_k_wgs": r.sk_wgs, "strip_rows": r.strip_rows,
            "kernel_ms_mean": round(gpu_ms, 5), "kernel_us_mean": round(gpu_ms * 1e3, 2),
            "timing": "HIP events on the launch stream around the timed region, per step",
            "entry": r.entry, "workspace_bytes": r.ws_bytes,
            "library_digest": library_digest()}


def cpu_baseline(p, first_out: np.ndarray, seconds: float):
    """Oracle on the first J columns of problem p; also checks the GPU's first
    output on those columns."""
    import oracle
    oracle.build(force=False)
    cores = oracle.num_threads()
    if p.rowmajor:
        raise ValueError("cpu baseline is defined for the column-major workloads")

    def run(cols):
        t0 = time.perf_counter()
        R = oracle.gemm(p.m, cols, p.k, p.alpha, p.A, p.lda, p.B, p.ldb, p.beta, p.C, p.ldc,
                        dtype=p.dtype)
        return R, time.perf_counter() - t0

    probe = min(p.n, first_out.shape[1], 16)
    _, tp = run(probe)
    cols = int(min(p.n, first_out.shape[1], max(probe, probe * seconds / max(tp, 1e-6))))
    R, dt = run(cols)
    flops = 2.0 * p.m * cols * p.k
    got = first_out[:, :cols].astype(np.float64)
    D = got - R
    rel = float(np.linalg.norm(D) / np.linalg.norm(R))
    maxabs = float(np.max(np.abs(D)))
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOPS", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": "first %d of %d columns of C (%dx%dx%d, %.1f GFLOP), OMP threads=%d, "
                      "affinity cpus=%d" % (cols, p.n, p.m, cols, p.k, flops / 1e9, cores,
                                            len(os.sched_getaffinity(0))),
            "sample_parity": {"max_abs": maxabs, "rel_fro": rel,
                              "ok": bool(maxabs <= 1e-6 * p.k and rel <= 1e-5)}}


def sweep(args):
    """Every workload: GPU time per call (two HIP events on the launch stream
    around a run of back-to-back launches, about 50 ms of GPU time), the
    parity figures against the oracle (full result up to 4096^3, the first
    columns at 8192^3) and the oracle's time on the same columns."""
    import torch
    import oracle
    oracle.build(force=False)
    cores = oracle.num_threads()
    rows = []
    # written between the launches of the cold-cache timing: twice the
    # 256 MB MALL, so no operand survives in any cache
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    one_thread = {}
    for name in gi.WORKLOADS:
        log("sweep", name)
        r = Resident(name)
        p = r.p
        r.launch()
        torch.cuda.synchronize()
        if p.rowmajor:
            out = r.C.cpu().numpy()
            got = gi.logical_rowmajor(out, p.m, p.n, p.ldc).astype(np.float64)
        else:
            out = r.C.cpu().numpy()
            got = gi.logical_colmajor(out, p.m, p.n, p.ldc).astype(np.float64)
        r.reset_c()
        _, per = warm_up(r, args.warmup, args.min_warmup_seconds)
        _, kern_ms = timed_steps(r, auto_steps(r, max(args.steps, 10), per))
        cold_ms = cold_kernel_ms(r, flush, 5)
        cols = p.n if p.m * p.n * p.k <= 4096 ** 3 else 512
        t0 = time.perf_counter()
        if p.rowmajor:
            R = oracle.matmat_rowmajor_f64(p.lda, p.ldb, p.ldc, p.A, p.B, p.C, p.m, p.k, p.n)
        else:
            R = oracle.gemm(p.m, cols, p.k, p.alpha, p.A, p.lda, p.B, p.ldb, p.beta, p.C,
                            p.ldc, dtype=p.dtype)
        t_or = time.perf_counter() - t0
        if name in ONE_THREAD_WORKLOADS:
            oracle.set_num_threads(1)
            t1 = time.perf_counter()
            oracle.gemm(p.m, cols, p.k, p.alpha, p.A, p.lda, p.B, p.ldb, p.beta, p.C, p.ldc,
                        dtype=p.dtype)
            one_thread[name] = time.perf_counter() - t1
            oracle.set_num_threads(cores)
        D = got[:, :cols] - R
        maxabs = float(np.max(np.abs(D)))
        rel = float(np.linalg.norm(D) / np.linalg.norm(R))
        if r.dt == "f32":
            ok = maxabs <= 1e-6 * p.k and rel <= 1e-5
        else:
            ok = rel <= 1e-12
        cnt = recorded_counters(r.variant, r.name)
        tflops = r.flops / (kern_ms * 1e-3) / 1e12
        rows.append((name, "%dx%dx%d" % (p.m, p.n, p.k), r.entry, r.variant, kern_ms, tflops,
                     100 * tflops / PEAK_TFLOPS[r.dt], cnt, maxabs, rel, ok, t_or, cols, p.n,
                     2.0 * p.m * cols * p.k / t_or / 1e9, cold_ms,
                     100 * tflops / device_peak(r.dt)[0]))
        del r
        torch.cuda.empty_cache()
    print("| workload | M×N×K | entry, variant | GPU ms per call | TFLOP/s | %% of peak "
          "(device props) | cold-cache ms | MfmaUtil | LDS bank conflicts | max\\|ΔC\\| "
          "| rel. Frobenius | parity | oracle s (%d threads) | oracle GFLOP/s |" % cores)
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for (name, shape, entry, var, ms, tf, pct, cnt, maxabs, rel, ok, t_or, cols, n,
         ogf, cold, dpct) in rows:
        mu = "%.1f %%" % (100 * cnt["mfma_util"]) if cnt else "—"
        lc = "%d" % cnt["lds_bank_conflict_cycles"] if cnt else "—"
        part = "" if cols == n else " (first %d of %d columns)" % (cols, n)
        print("| %s | %s | `%s`, %s | %.4f | %.1f | %.1f (%.1f) | %.4f | %s | %s | %.3g | %.3g "
              "| %s | %.2f%s | %.1f |" % (name, shape, entry, var, ms, tf, pct, dpct, cold, mu,
                                          lc, maxabs, rel, "pass" if ok else "FAIL", t_or,
                                          part, ogf))
    dpeak, cus, mhz = device_peak("f32")
    print("\nDevice properties: %d compute units at %.0f MHz, fp32 matrix peak %.1f TFLOP/s "
          "(fp64 %.1f)." % (cus, mhz, dpeak, dpeak / 2))
    for name, t1 in one_thread.items():
        p = gi.workload(name)
        print("Oracle on 1 thread, %s: %.3f s (%.2f GFLOP/s)." %
              (name, t1, 2.0 * p.m * p.n * p.k / t1 / 1e9))
    sys.stdout.flush()


# workloads whose oracle is also timed on one thread (for scale)
ONE_THREAD_WORKLOADS = ("sgemm_128", "sgemm_2048")


def cold_kernel_ms(r: Resident, flush, launches: int) -> float:
    """Median kernel time with cold caches: before each launch, outside its
    pair of HIP events, C is restored (beta != 0) and a 512 MiB buffer is
    written, which evicts the operands from L2 and the MALL."""
    import torch
    times = []
    for t in range(launches):
        r.reset_c()
        flush.fill_(t & 0xFF)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(r.stream)
        r.launch()
        e.record(r.stream)
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    r.reset_c()
    return float(np.median(times))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the GEMM is not sharded across GPUs in this "
              "library (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.sweep:
        sweep(args)
        return

    log("generating", args.workload)
    r = Resident(args.workload)
    log("variant", r.variant)
    # first call on the pristine C: kept for the CPU sample check
    r.launch()
    torch.cuda.synchronize()
    first_out = None
    if not args.no_cpu_baseline and not r.p.rowmajor:
        p = r.p
        first_out = r.C[: p.ldc * p.n].view(p.n, p.ldc)[:, : p.m].t().cpu().numpy()
    r.reset_c()
    n_warm, _ = warm_up(r, args.warmup, args.min_warmup_seconds)
    ms_step, gpu_ms = timed_steps(r, args.steps)
    value = r.flops / (ms_step * 1e-3) / 1e12
    log("%s: %.3f ms/step wall, %.3f ms/step GPU -> %.2f TFLOPS" % (r.name, ms_step, gpu_ms,
                                                                    value))
    p = r.p
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_launches": n_warm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": r.dt, "data": "synthetic",
        "config": {"workload": r.name, "m": p.m, "n": p.n, "k": p.k, "lda": p.lda,
                   "ldb": p.ldb, "ldc": p.ldc, "alpha": p.alpha, "beta": p.beta,
                   "layout": "row-major (operand swap)" if p.rowmajor else "column-major",
                   "variant": r.variant, "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / PEAK_TFLOPS[r.dt], 2),
        "roofline": roofline(r, gpu_ms),
    }
    main_problem = r.p
    secondary = []
    for name in args.secondary:
        if name == args.workload:
            continue
        del r
        torch.cuda.empty_cache()
        r2 = Resident(name)
        nw2, per = warm_up(r2, args.warmup, args.min_warmup_seconds)
        steps2 = auto_steps(r2, max(args.steps, 20), per)
        ms2, g2 = timed_steps(r2, steps2)
        v2 = r2.flops / (ms2 * 1e-3) / 1e12
        log("%s: %.4f ms/step wall, %.4f ms/step GPU (%d steps) -> %.2f TFLOPS" % (
            name, ms2, g2, steps2, v2))
        secondary.append({"workload": name, "value": round(v2, 3), "unit": "TFLOPS",
                          "ms_per_step": round(ms2, 5), "us_per_step": round(ms2 * 1e3, 2),
                          "steps": steps2, "warmup_launches": nw2, "dtype": r2.dt,
                          "pct_of_peak": round(100 * v2 / PEAK_TFLOPS[r2.dt], 2),
                          "roofline": roofline(r2, g2)})
        r = r2
    if secondary:
        out["secondary"] = secondary
    if args.calibrate_copy_mib > 0:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = nbytes
        del src, dst
    if first_out is not None:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(main_problem, first_out, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
