"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The CPU oracle (``oracle/oracle.c``) is built with gcc's
  ``-fsanitize=address,undefined`` and runs every pin of ``oracle_pins.py``
  in a child process with the sanitizer runtimes preloaded: an out-of-bounds
  index or an integer overflow in the oracle would abort it.
* The library's host side (argument checks, the tile-class choice, the
  stream-K plan, the strip rows, the workspace sizes) is built by hipcc
  with the same sanitizers on the host pass only, and a child process
  drives the selection and workspace entry points over seeded random shapes
  up to 2^31 - 1 per dimension, plus the argument-error returns.  None of
  these calls reaches the GPU: no kernel is launched.

Each test is skipped when its compiler or sanitizer runtime is missing.
"""
import glob
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "precision_gemm_02_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "4"}


def _gcc_runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if shutil.which("gcc") is None or asan is None or ubsan is None:
        pytest.skip("gcc with libasan/libubsan is not available")
    so = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-std=c11", "-shared", "-fPIC", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", so,
                    os.path.join(ROOT, "oracle", "oracle.c")], check=True)
    proc = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), so],
                          capture_output=True, text=True, timeout=600,
                          env={**os.environ, **ENV, "LD_PRELOAD": asan + " " + ubsan})
    assert proc.returncode == 0, (proc.stdout[-3000:], proc.stderr[-3000:])
    assert "PIN-FAILED" not in proc.stdout


DRIVER = textwrap.dedent("""
    import ctypes, random, sys
    L = ctypes.CDLL(sys.argv[1])
    i, f, d, vp, sz = ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER(i)
    L.pgemm_select_ws_f32.argtypes = [i, i, i, f, vp, i, vp, i, f, vp, i, sz, P, P]
    L.pgemm_select_ws_f64.argtypes = [i, i, i, d, vp, i, vp, i, d, vp, i, sz, P, P]
    L.pgemm_select_f32.argtypes = [i, i, i, f, vp, i, vp, i, f, vp, i]
    L.pgemm_workspace_f32.restype = sz
    L.pgemm_workspace_f64.restype = sz
    L.pgemm_workspace_f32.argtypes = [i, i, i]
    L.pgemm_workspace_f64.argtypes = [i, i, i]
    L.gemm_f32.argtypes = [i, i, i, f, vp, i, vp, i, f, vp, i, vp]
    L.gemm_f32_noalloc.argtypes = L.gemm_f32.argtypes
    L.gemm_f64.argtypes = [i, i, i, d, vp, i, vp, i, d, vp, i, vp]
    L.matmat_f64.argtypes = [i, i, i, vp, vp, vp, i, i, i, vp]
    L.pgemm_matmat_host_workspace.restype = sz
    L.pgemm_matmat_host_workspace.argtypes = [i, i, i, i, i, i]
    L.pgemm_status_string.restype = ctypes.c_char_p
    L.pgemm_variant_name.restype = ctypes.c_char_p
    rng = random.Random(int(sys.argv[2]))
    F, TOP = 1 << 20, (1 << 31) - 1
    for t in range(int(sys.argv[3])):
        hi = TOP if rng.random() < 0.2 else 20000
        m, n, k = (rng.randint(0, hi) for _ in range(3))
        lda = min(max(1, m) + rng.randint(0, 3), TOP)
        ldb = min(max(1, k) + rng.randint(0, 3), TOP)
        for dt in (32, 64):
            ws = (L.pgemm_workspace_f32 if dt == 32 else L.pgemm_workspace_f64)(m, n, k)
            sk, strip = i(0), i(0)
            sel = L.pgemm_select_ws_f32 if dt == 32 else L.pgemm_select_ws_f64
            v = sel(m, n, k, 1.0, F, lda, F, ldb, 0.5, F, lda, ws if t % 2 else 0,
                    ctypes.byref(sk), ctypes.byref(strip))
            assert v >= 0 and 0 <= strip.value <= 8 and sk.value >= 0, (m, n, k, v)
            if v > 0:
                assert L.pgemm_variant_name(v) is not None
        L.pgemm_matmat_host_workspace(lda, ldb, lda, m, n, k)
        # argument errors return before any HIP call
        assert L.gemm_f32(-1, n, k, 1.0, F, 1, F, 1, 0.0, F, 1, None) == -1
        assert L.gemm_f32_noalloc(m, n, -1, 1.0, F, 1, F, 1, 0.0, F, 1, None) == -3
        if m > 1:
            assert L.gemm_f64(m, n, k, 1.0, F, m - 1, F, max(1, k), 0.0, F, m, None) == -6
        assert L.matmat_f64(0, 1, 1, F, F, F, 4, 4, 4, None) == -1
    for s in (0, -1, -6, -100, -101, -102, 12345):
        assert L.pgemm_status_string(s)
    print("ok")
""")


def test_library_host_logic_under_asan_and_ubsan(tmp_path):
    hipcc = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
    runtimes = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not os.path.exists(hipcc) or not runtimes:
        pytest.skip("hipcc or its address-sanitizer runtime is not available")
    import concurrent.futures

    def compile_one(src):
        # the device code is built as usual (its kernels are never launched
        # here); only the host pass is instrumented
        obj = str(tmp_path / src.replace(".hip", ".o"))
        proc = subprocess.run(
            [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + CSRC, "-I" + INCLUDE,
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-c", os.path.join(CSRC, src), "-o", obj], capture_output=True, text=True)
        assert proc.returncode == 0, proc.stderr[-3000:]
        return obj

    with concurrent.futures.ThreadPoolExecutor(3) as ex:
        objs = list(ex.map(compile_one, ("api.hip", "sgemm.hip", "dgemm.hip")))
    so = str(tmp_path / "libpgemm_san.so")
    proc = subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC",
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                           "-fsanitize=undefined", "-shared-libsan", "-o", so, *objs],
                          capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-3000:]
    driver = tmp_path / "drive.py"
    driver.write_text(DRIVER)
    proc = subprocess.run([sys.executable, str(driver), so, "7", "20000"], capture_output=True,
                          text=True, timeout=600,
                          env={**os.environ, **ENV, "LD_PRELOAD": runtimes[0]})
    assert proc.returncode == 0 and proc.stdout.strip().endswith("ok"), (
        proc.stdout[-3000:], proc.stderr[-3000:])
