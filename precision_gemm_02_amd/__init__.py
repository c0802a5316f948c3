"""pgemm: C <- alpha*A*B + beta*C on AMD MI355X (gfx950), fp32 and fp64.

Thin ctypes binding over ``libpgemm.so`` (the C ABI declared in
``include/pgemm.h``).  Every step of the computation runs in the library's
HIP kernels; this module only turns tensors or integer device addresses into
pointers, leading dimensions and a stream handle.  PyTorch is used only for
device memory and the current stream.

Functions with the C names take the C arguments (A, B, C may be torch tensors
on the GPU or integer device addresses; ``stream`` defaults to torch's
current stream).  ``gemm(A, B, C, alpha, beta)`` takes 2-D tensors and reads
the layout from their strides: a column-major view (stride (1, ld)) is used
as is; a row-major tensor (stride (ld, 1)) is served by the operand swap
C^T = B^T A^T, which moves no data.

The library must be built (``python precision_gemm_02_amd/build.py``, which
does not import this package); if it is missing or older than this binding,
importing this package raises ImportError.  There is no CPU or
eager fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpgemm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libpgemm.so is not built; run `python precision_gemm_02_amd/build.py` "
                      "(or __graft_entry__.build()) first")

# PyTorch-ROCm ships its own HIP runtime with the same SONAME as the system
# one (libamdhip64.so.7).  Loading torch first makes the dynamic linker bind
# libpgemm.so to that already-loaded runtime, so that device pointers and
# stream handles from torch are valid in the library.  Two runtimes in one
# process would make every torch stream handle foreign to the library.
import torch as _torch  # noqa: E402,F401  (load order matters)


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


_lib = ctypes.CDLL(LIB_PATH)
if len(_hip_runtimes_mapped()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process (%s); import torch before "
                      "anything that loads /opt/rocm's libamdhip64" %
                      ", ".join(sorted(_hip_runtimes_mapped())))

# every entry point include/pgemm.h declares
_EXPORTS = ("gemm_f32", "gemm_f64", "matmat_f64", "pgemm_status_string",
            "pgemm_select_f32", "pgemm_select_f64", "pgemm_variant_name",
            "pgemm_num_variants", "gemm_f32_variant", "gemm_f64_variant",
            "gemm_f32_ws", "gemm_f64_ws", "pgemm_workspace_f32", "pgemm_workspace_f64",
            "matmat_f64_host", "pgemm_matmat_host_workspace", "pgemm_select_ws_f32",
            "pgemm_select_ws_f64", "pgemm_device_info", "gemm_f32_noalloc")
_missing = [n for n in _EXPORTS if not hasattr(_lib, n)]
if _missing:
    raise ImportError("libpgemm.so is older than this binding (no %s); rebuild it with "
                      "`python precision_gemm_02_amd/build.py`" % ", ".join(_missing))

_i, _f, _d, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
_lib.gemm_f32.argtypes = [_i, _i, _i, _f, _vp, _i, _vp, _i, _f, _vp, _i, _vp]
_lib.gemm_f64.argtypes = [_i, _i, _i, _d, _vp, _i, _vp, _i, _d, _vp, _i, _vp]
_lib.matmat_f64.argtypes = [_i, _i, _i, _vp, _vp, _vp, _i, _i, _i, _vp]
_lib.gemm_f32_variant.argtypes = [_i] + _lib.gemm_f32.argtypes
_lib.gemm_f64_variant.argtypes = [_i] + _lib.gemm_f64.argtypes
_lib.pgemm_select_f32.argtypes = [_i, _i, _i, _f, _vp, _i, _vp, _i, _f, _vp, _i]
_lib.pgemm_select_f64.argtypes = [_i, _i, _i, _d, _vp, _i, _vp, _i, _d, _vp, _i]
_sz = ctypes.c_size_t
_lib.pgemm_select_ws_f32.argtypes = _lib.pgemm_select_f32.argtypes + [_sz, ctypes.POINTER(_i),
                                                                       ctypes.POINTER(_i)]
_lib.pgemm_select_ws_f64.argtypes = _lib.pgemm_select_f64.argtypes + [_sz, ctypes.POINTER(_i),
                                                                       ctypes.POINTER(_i)]
_lib.gemm_f32_ws.argtypes = _lib.gemm_f32.argtypes[:11] + [_vp, _sz, _vp]
_lib.gemm_f32_noalloc.argtypes = _lib.gemm_f32.argtypes
_lib.gemm_f64_ws.argtypes = _lib.gemm_f64.argtypes[:11] + [_vp, _sz, _vp]
_lib.pgemm_workspace_f32.argtypes = [_i, _i, _i]
_lib.pgemm_workspace_f64.argtypes = [_i, _i, _i]
_lib.pgemm_workspace_f32.restype = _sz
_lib.pgemm_workspace_f64.restype = _sz
_lib.matmat_f64_host.argtypes = [_i, _i, _i, _vp, _vp, _vp, _i, _i, _i, _vp, _sz, _vp]
_lib.matmat_f64_host.restype = _i
_lib.pgemm_matmat_host_workspace.argtypes = [_i, _i, _i, _i, _i, _i]
_lib.pgemm_matmat_host_workspace.restype = _sz
_lib.pgemm_status_string.argtypes = [_i]
_lib.pgemm_status_string.restype = ctypes.c_char_p
_lib.pgemm_variant_name.argtypes = [_i]
_lib.pgemm_variant_name.restype = ctypes.c_char_p
for _name in ("gemm_f32", "gemm_f64", "matmat_f64", "gemm_f32_variant", "gemm_f64_variant",
              "pgemm_select_f32", "pgemm_select_f64", "pgemm_num_variants", "gemm_f32_ws",
              "gemm_f64_ws", "pgemm_select_ws_f32", "pgemm_select_ws_f64",
              "pgemm_device_info", "gemm_f32_noalloc"):
    getattr(_lib, _name).restype = _i
_lib.pgemm_device_info.argtypes = [ctypes.POINTER(_i), ctypes.POINTER(_i)]

PGEMM_OK = 0
PGEMM_EHIP = -100
PGEMM_EVARIANT = -101
PGEMM_ESCRATCH = -102
PGEMM_SCRATCH_BYTES = 32 << 20

EXPORTS = _EXPORTS


class PgemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: status %d (%s)" % (where, status, status_string(status)))
        self.status = status


def library():
    """The loaded ctypes library (for callers that want raw status codes)."""
    return _lib


def status_string(status: int) -> str:
    return _lib.pgemm_status_string(status).decode()


def _addr(x):
    """Device address of a tensor (its data pointer) or an int; None -> NULL.

    A tensor must live on the current HIP device: the kernels dereference
    the address on the GPU, where a host address (a CPU tensor's) or another
    device's memory would be a memory-access fault, not an error code.  An
    int is taken as a device address as is."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    dev = getattr(x, "device", None)
    if dev is None:
        raise TypeError("expected a torch tensor, an int device address or None, got %s"
                        % type(x).__name__)
    if dev.type != "cuda":
        raise TypeError("tensor is on %s; pgemm needs device (HIP) memory" % dev)
    import torch
    if dev.index != torch.cuda.current_device():
        raise TypeError("tensor is on %s but the current device is cuda:%d"
                        % (dev, torch.cuda.current_device()))
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where):
    if status != PGEMM_OK:
        raise PgemmError(status, where)


def gemm_f32(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """C <- alpha*A*B + beta*C, fp32, column-major (see include/pgemm.h)."""
    _check(_lib.gemm_f32(m, n, k, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                         _stream(stream)), "gemm_f32")


def gemm_f64(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """C <- alpha*A*B + beta*C, fp64, column-major (see include/pgemm.h)."""
    _check(_lib.gemm_f64(m, n, k, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                         _stream(stream)), "gemm_f64")


def matmat_f64(lda, ldb, ldc, A, B, C, N1, N2, N3, stream=None):
    """Row-major C(N1 x N3) += A(N1 x N2) * B(N2 x N3), fp64 (lecture form)."""
    _check(_lib.matmat_f64(lda, ldb, ldc, _addr(A), _addr(B), _addr(C), N1, N2, N3,
                           _stream(stream)), "matmat_f64")


def gemm_f32_ws(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, ws, ws_bytes, stream=None):
    """gemm_f32 with a device workspace for balancing leftover tiles."""
    _check(_lib.gemm_f32_ws(m, n, k, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                            _addr(ws), ws_bytes, _stream(stream)), "gemm_f32_ws")


def gemm_f64_ws(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, ws, ws_bytes, stream=None):
    """gemm_f64 with a device workspace for balancing leftover tiles."""
    _check(_lib.gemm_f64_ws(m, n, k, alpha, _addr(A), lda, _addr(B), ldb, beta, _addr(C), ldc,
                            _addr(ws), ws_bytes, _stream(stream)), "gemm_f64_ws")


def gemm_f32_noalloc(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    """gemm_f32_ws on the library's own fixed scratch array (allocates
    nothing; calls on one device must be ordered)."""
    _check(_lib.gemm_f32_noalloc(m, n, k, alpha, _addr(A), lda, _addr(B), ldb, beta,
                                 _addr(C), ldc, _stream(stream)), "gemm_f32_noalloc")


def workspace_f32(m, n, k) -> int:
    """Workspace bytes gemm_f32_ws can use for this shape (0: none)."""
    return _lib.pgemm_workspace_f32(m, n, k)


def workspace_f64(m, n, k) -> int:
    return _lib.pgemm_workspace_f64(m, n, k)


def _host_addr(x):
    """Host address of a numpy array (its data pointer) or an int; None -> NULL."""
    if x is None or isinstance(x, int):
        return x
    if not x.flags["C_CONTIGUOUS"] and not x.flags["F_CONTIGUOUS"]:
        raise ValueError("host arrays must be contiguous storage")
    return x.ctypes.data


def matmat_f64_host(lda, ldb, ldc, A, B, C, N1, N2, N3, ws, ws_bytes, stream=None):
    """Lecture matmat (row-major, C += A*B) on host arrays (numpy float64
    storage or int addresses) with a device workspace; returns when C is back
    in host memory."""
    _check(_lib.matmat_f64_host(lda, ldb, ldc, _host_addr(A), _host_addr(B), _host_addr(C),
                                N1, N2, N3, _addr(ws), ws_bytes, _stream(stream)),
           "matmat_f64_host")


def matmat_host_workspace(lda, ldb, ldc, N1, N2, N3) -> int:
    """Device workspace bytes matmat_f64_host needs."""
    return _lib.pgemm_matmat_host_workspace(lda, ldb, ldc, N1, N2, N3)


def gemm_f32_variant(variant, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    _check(_lib.gemm_f32_variant(variant, m, n, k, alpha, _addr(A), lda, _addr(B), ldb, beta,
                                 _addr(C), ldc, _stream(stream)), "gemm_f32_variant")


def gemm_f64_variant(variant, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream=None):
    _check(_lib.gemm_f64_variant(variant, m, n, k, alpha, _addr(A), lda, _addr(B), ldb, beta,
                                 _addr(C), ldc, _stream(stream)), "gemm_f64_variant")


def select_f32(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc) -> int:
    return _lib.pgemm_select_f32(m, n, k, alpha, _addr(A), lda, _addr(B), ldb, beta,
                                 _addr(C), ldc)


def select_f64(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc) -> int:
    return _lib.pgemm_select_f64(m, n, k, alpha, _addr(A), lda, _addr(B), ldb, beta,
                                 _addr(C), ldc)


def select_ws_f32(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, ws_bytes):
    """(variant id, stream-K workgroups, strip rows) gemm_f32_ws would use."""
    sk, strip = ctypes.c_int(0), ctypes.c_int(0)
    v = _lib.pgemm_select_ws_f32(m, n, k, alpha, _addr(A), lda, _addr(B), ldb, beta,
                                 _addr(C), ldc, ws_bytes, ctypes.byref(sk), ctypes.byref(strip))
    return v, sk.value, strip.value


def select_ws_f64(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, ws_bytes):
    """(variant id, stream-K workgroups, strip rows) gemm_f64_ws would use."""
    sk, strip = ctypes.c_int(0), ctypes.c_int(0)
    v = _lib.pgemm_select_ws_f64(m, n, k, alpha, _addr(A), lda, _addr(B), ldb, beta,
                                 _addr(C), ldc, ws_bytes, ctypes.byref(sk), ctypes.byref(strip))
    return v, sk.value, strip.value


def device_info():
    """(compute units, peak clock in kHz) of the current device."""
    cus, khz = ctypes.c_int(0), ctypes.c_int(0)
    _check(_lib.pgemm_device_info(ctypes.byref(cus), ctypes.byref(khz)), "pgemm_device_info")
    return cus.value, khz.value


def variants():
    """{id: name} of every compiled kernel variant."""
    out = {}
    for v in range(1, _lib.pgemm_num_variants() + 1):
        out[v] = _lib.pgemm_variant_name(v).decode()
    return out


def _layouts(t):
    """{layout: ld} of every layout a 2-D tensor's strides fit: 'col'
    (element (i, j) at i + j*ld) and/or 'row' (at i*ld + j).  A dimension of
    size 1 has no stride to speak of, so a column (r x 1) fits column-major
    with ld = r and row-major with ld = 1 alike; callers take the layout
    the other operands agree on."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    r, c = t.shape
    s0, s1 = t.stride()
    out = {}
    if (r <= 1 or s0 == 1) and (c <= 1 or s1 >= max(1, r)):
        out["col"] = s1 if c > 1 else max(1, r)
    if (c <= 1 or s1 == 1) and (r <= 1 or s0 >= max(1, c)):
        out["row"] = s0 if r > 1 else max(1, c)
    if not out:
        raise ValueError("tensor with strides %s is neither column- nor row-major"
                         % (t.stride(),))
    return out


def gemm(A, B, C, alpha=1.0, beta=0.0, stream=None):
    """C <- alpha*A@B + beta*C in place, for GPU tensors of one dtype.

    All three tensors must share one layout: column-major views (e.g.
    ``X.t().contiguous().t()`` or a slice of one with padding) or row-major
    (contiguous) tensors.  Row-major uses the operand swap C^T = B^T A^T.
    """
    import torch
    if not (A.dtype == B.dtype == C.dtype) or A.dtype not in (torch.float32, torch.float64):
        raise TypeError("A, B, C must all be float32 or all float64")
    m, k = A.shape
    k2, n = B.shape
    if k2 != k or tuple(C.shape) != (m, n):
        raise ValueError("shape mismatch: A %s, B %s, C %s" % (tuple(A.shape), tuple(B.shape),
                                                              tuple(C.shape)))
    for name, t in (("A", A), ("B", B), ("C", C)):
        _addr(t)   # on the current device (TypeError otherwise)
    la, lb, lc = _layouts(A), _layouts(B), _layouts(C)
    fn = gemm_f32 if A.dtype == torch.float32 else gemm_f64
    if "col" in la and "col" in lb and "col" in lc:
        fn(m, n, k, alpha, A, la["col"], B, lb["col"], beta, C, lc["col"], stream)
    elif "row" in la and "row" in lb and "row" in lc:
        fn(n, m, k, alpha, B, lb["row"], A, la["row"], beta, C, lc["row"], stream)
    else:
        raise ValueError("A, B and C must share one layout")
    return C
