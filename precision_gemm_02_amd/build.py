"""Build libpgemm.so from csrc/ with hipcc for gfx950.

Each .hip file is compiled to an object in parallel, then linked into one
shared library next to this file.  Usage: ``python precision_gemm_02_amd/build.py``
(run as a file, it does not import the package, whose import needs a
current library).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libpgemm.so")
SOURCES = ["api.hip", "sgemm.hip", "dgemm.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=fast",
    # never emit packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + CSRC, "-I" + INCLUDE,
    "-Wall", "-Wno-unused-result",
]


def source_digest(extra_flags=()) -> str:
    """sha256 (first 16 hex digits) of what determines the built kernels: the
    compiler flags and the bytes of every file under csrc/ and of the public
    header.  Unlike a hash of libpgemm.so it does not depend on the directory
    the library is built in (hipcc derives per-file symbols from the path)."""
    import hashlib
    h = hashlib.sha256()
    h.update(" ".join([ARCH, *[f for f in CFLAGS if not f.startswith("-I")],
                       *extra_flags]).encode())
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC))
    files.append(os.path.join(INCLUDE, "pgemm.h"))
    for path in files:
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in proc.stderr.splitlines() if noise not in ln)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(extra_flags=()) -> str:
    """Compile every kernel source for gfx950 and link libpgemm.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("link failed:\n" + proc.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(sys.argv[1:]))
