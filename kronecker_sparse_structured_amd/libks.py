"""Thin Python binding of libks (include/ks.h) through ctypes.

The functions named like the C entry points (``ks_matmul``, ``ks_matmul_ex``,
``ks_chain_workspace_size``, ``ks_chain_matmul``, ``ks_chain_plan``,
``ks_chain_describe``, ``ks_plan_describe``, ``ks_status_string``,
``ks_version``, the gradient calls) only marshal arguments: tensors become
device pointers, the stream defaults to torch's current stream, and a
non-OK status raises ``KSError``. Every step of the computation runs in the
HIP kernels of libks.so; there is no fallback. If the library is not built,
loading fails loudly.

``matmul`` and ``chain_matmul`` are conveniences over the same calls that
allocate the output (and the chain workspace) with torch.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libks.so")

# ks_dtype_t
DTYPE_F32, DTYPE_BF16, DTYPE_BF16W = 0, 1, 2
# ks_kernel_t
KERNEL_AUTO, KERNEL_GENERIC, KERNEL_VALU, KERNEL_MFMA, KERNEL_MFMA_LDS, KERNEL_COLUMN = 0, 1, 2, 3, 4, 5
KERNELS = {"auto": KERNEL_AUTO, "generic": KERNEL_GENERIC, "valu": KERNEL_VALU, "mfma": KERNEL_MFMA,
           "mfma_lds": KERNEL_MFMA_LDS, "col": KERNEL_COLUMN}
# ks_store_waves_t
STORE_AUTO, STORE_COMPUTE, STORE_DEDICATED = 0, 1, 2
STORE_WAVES = {"auto": STORE_AUTO, "compute": STORE_COMPUTE, "dedicated": STORE_DEDICATED}
# chain flags
CHAIN_AUTO, CHAIN_NO_FUSE = 0, 1
# ks_status_t
STATUS = ["KS_OK", "KS_ERR_NULL", "KS_ERR_PATTERN", "KS_ERR_BATCH", "KS_ERR_DTYPE",
          "KS_ERR_CHAIN_MISMATCH", "KS_ERR_WORKSPACE", "KS_ERR_ALIGN", "KS_ERR_OVERLAP",
          "KS_ERR_HIP", "KS_ERR_UNSUPPORTED", "KS_ERR_INVALID"]
for _i, _n in enumerate(STATUS):
    globals()[_n] = _i


class KSError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, ks_status_string(status)))


class ks_pattern_t(ctypes.Structure):
    _fields_ = [("a", ctypes.c_int32), ("b", ctypes.c_int32),
                ("c", ctypes.c_int32), ("d", ctypes.c_int32)]


MFMA_TILES = 7   # KS_MFMA_TILES: tile candidates of the matrix-core kernel


class ks_options_t(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("rows_per_block", ctypes.c_int32),
                ("store_waves", ctypes.c_int32), ("mfma_tile", ctypes.c_int32), ("mfma_loaders", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 3)]


class ks_closure_t(ctypes.Structure):
    _fields_ = [("components", ctypes.c_int64), ("mid", ctypes.c_int64), ("inputs", ctypes.c_int64),
                ("outputs", ctypes.c_int64), ("weights", ctypes.c_int64), ("in_run", ctypes.c_int64),
                ("out_run", ctypes.c_int64), ("tile_components", ctypes.c_int64), ("tile_weights", ctypes.c_int64),
                ("uniform", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib = None


def _hip_runtimes() -> set:
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return {line.split()[-1] for line in f
                    if len(line.split()) >= 6 and "libamdhip64.so" in line.split()[-1]}
    except OSError:
        return set()


def load(path: str = LIB_PATH):
    """Load libks.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            "libks.so not found at %s; build it with "
            "`python -m kronecker_sparse_structured_amd.build`" % path)
    # torch ships its own copy of the HIP runtime. Load it first so that
    # libks binds to that copy: with two runtimes in one process, pointers
    # and streams from torch are unknown to the one libks calls.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise RuntimeError("more than one HIP runtime is loaded in this process (%s); "
                           "libks must share torch's" % ", ".join(sorted(runtimes)))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.ks_status_string.argtypes = [i32]
    lib.ks_status_string.restype = ctypes.c_char_p
    lib.ks_version.argtypes = []
    lib.ks_version.restype = ctypes.c_char_p
    lib.ks_matmul.argtypes = [ks_pattern_t, vp, vp, vp, i64, i32, vp]
    lib.ks_matmul.restype = i32
    lib.ks_matmul_ex.argtypes = [ks_pattern_t, vp, vp, vp, i64, i32, vp, ctypes.POINTER(ks_options_t)]
    lib.ks_matmul_ex.restype = i32
    lib.ks_chain_workspace_size.argtypes = [ctypes.POINTER(ks_pattern_t), i32, i64, i32,
                                            ctypes.c_uint, ctypes.POINTER(ctypes.c_size_t)]
    lib.ks_chain_workspace_size.restype = i32
    lib.ks_chain_matmul.argtypes = [ctypes.POINTER(ks_pattern_t), i32, ctypes.POINTER(vp), vp, vp,
                                    i64, i32, vp, ctypes.c_size_t, ctypes.c_uint, vp]
    lib.ks_chain_matmul.restype = i32
    lib.ks_chain_plan.argtypes = [ctypes.POINTER(ks_pattern_t), i32, i64, i32, ctypes.c_uint,
                                  ctypes.POINTER(ctypes.c_int), i32, ctypes.POINTER(ctypes.c_int)]
    lib.ks_chain_plan.restype = i32
    lib.ks_plan_describe.argtypes = [ks_pattern_t, i64, i32, ctypes.c_char_p, ctypes.c_size_t]
    lib.ks_plan_describe.restype = i32
    lib.ks_chain_describe.argtypes = [ctypes.POINTER(ks_pattern_t), i32, i64, i32, ctypes.c_uint,
                                      ctypes.c_char_p, ctypes.c_size_t]
    lib.ks_chain_describe.restype = i32
    lib.ks_pair_closure.argtypes = [ks_pattern_t, ks_pattern_t, ctypes.POINTER(ks_closure_t)]
    lib.ks_pair_closure.restype = i32
    lib.ks_matmul_dx_workspace_size.argtypes = [ks_pattern_t, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.ks_matmul_dx_workspace_size.restype = i32
    lib.ks_matmul_dx.argtypes = [ks_pattern_t, vp, vp, vp, i64, i32, vp, ctypes.c_size_t, vp]
    lib.ks_matmul_dx.restype = i32
    lib.ks_matmul_dw_workspace_size.argtypes = [ks_pattern_t, i64, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.ks_matmul_dw_workspace_size.restype = i32
    lib.ks_matmul_dw.argtypes = [ks_pattern_t, vp, vp, vp, i64, i32, vp, ctypes.c_size_t, vp]
    lib.ks_matmul_dw.restype = i32
    lib.ks_matmul_dw_noalloc.argtypes = [ks_pattern_t, vp, vp, vp, i64, i32, vp]
    lib.ks_matmul_dw_noalloc.restype = i32
    _lib = lib
    return lib


# ---------------------------------------------------------------- marshalling

def _pattern(p) -> ks_pattern_t:
    if isinstance(p, ks_pattern_t):
        return p
    a, b, c, d = (int(v) for v in p)
    return ks_pattern_t(a, b, c, d)


def _ptr(x) -> Optional[int]:
    """Device address of a tensor, or an int address, or None (NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream, *tensors) -> Optional[int]:
    if stream is None:
        import torch
        for t in tensors:
            if t is not None and not isinstance(t, int) and t.is_cuda:
                return int(torch.cuda.current_stream(t.device).cuda_stream)
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _raise(status: int, where: str, check: bool) -> int:
    if check and status != 0:
        raise KSError(status, where)
    return status


# ---------------------------------------------------------------- C entry points

def ks_status_string(status: int) -> str:
    return load().ks_status_string(int(status)).decode()


def ks_version() -> str:
    return load().ks_version().decode()


def ks_matmul(p, W, X, Y, batch: int, dtype: int, stream=None, check: bool = True) -> int:
    st = load().ks_matmul(_pattern(p), _ptr(W), _ptr(X), _ptr(Y), int(batch), int(dtype),
                          _stream(stream, Y, X, W))
    return _raise(st, "ks_matmul", check)


def ks_matmul_ex(p, W, X, Y, batch: int, dtype: int, stream=None, kernel: int = KERNEL_AUTO,
                 rows_per_block: int = 0, check: bool = True, reserved=None, store_waves=STORE_AUTO,
                 mfma_tile: int = 0, mfma_loaders: int = 0) -> int:
    opt = ks_options_t()
    opt.kernel = KERNELS.get(kernel, kernel) if isinstance(kernel, str) else int(kernel)
    opt.rows_per_block = int(rows_per_block)
    opt.mfma_tile = int(mfma_tile)
    opt.mfma_loaders = int(mfma_loaders)
    opt.store_waves = STORE_WAVES.get(store_waves, store_waves) if isinstance(store_waves, str) else int(store_waves)
    if reserved is not None:
        for i, v in enumerate(reserved):
            opt.reserved[i] = int(v)
    st = load().ks_matmul_ex(_pattern(p), _ptr(W), _ptr(X), _ptr(Y), int(batch), int(dtype),
                             _stream(stream, Y, X, W), ctypes.byref(opt))
    return _raise(st, "ks_matmul_ex", check)


def ks_matmul_dx_workspace_size(p, dtype: int, check: bool = True):
    out = ctypes.c_size_t(0)
    st = load().ks_matmul_dx_workspace_size(_pattern(p), int(dtype), ctypes.byref(out))
    _raise(st, "ks_matmul_dx_workspace_size", check)
    return out.value if check else (st, out.value)


def ks_matmul_dx(p, W, dY, dX, batch: int, dtype: int, ws, ws_bytes: int, stream=None, check: bool = True) -> int:
    st = load().ks_matmul_dx(_pattern(p), _ptr(W), _ptr(dY), _ptr(dX), int(batch), int(dtype), _ptr(ws),
                             int(ws_bytes), _stream(stream, dX, dY, W))
    return _raise(st, "ks_matmul_dx", check)


def ks_matmul_dw_workspace_size(p, batch: int, dtype: int, check: bool = True):
    out = ctypes.c_size_t(0)
    st = load().ks_matmul_dw_workspace_size(_pattern(p), int(batch), int(dtype), ctypes.byref(out))
    _raise(st, "ks_matmul_dw_workspace_size", check)
    return out.value if check else (st, out.value)


def ks_matmul_dw(p, dY, X, dW, batch: int, dtype: int, ws, ws_bytes: int, stream=None, check: bool = True) -> int:
    st = load().ks_matmul_dw(_pattern(p), _ptr(dY), _ptr(X), _ptr(dW), int(batch), int(dtype), _ptr(ws),
                             int(ws_bytes), _stream(stream, dW, dY, X))
    return _raise(st, "ks_matmul_dw", check)


def ks_matmul_dw_noalloc(p, dY, X, dW, batch: int, dtype: int, stream=None, check: bool = True) -> int:
    st = load().ks_matmul_dw_noalloc(_pattern(p), _ptr(dY), _ptr(X), _ptr(dW), int(batch), int(dtype),
                                     _stream(stream, dW, dY, X))
    return _raise(st, "ks_matmul_dw_noalloc", check)


def _patterns(ps: Sequence):
    arr = (ks_pattern_t * max(len(ps), 1))()
    for i, p in enumerate(ps):
        arr[i] = _pattern(p)
    return arr


def ks_chain_workspace_size(ps: Sequence, batch: int, dtype: int, flags: int = CHAIN_AUTO,
                            n: Optional[int] = None, check: bool = True):
    """Returns the workspace size in bytes (or (status, size) if check=False)."""
    out = ctypes.c_size_t(0)
    st = load().ks_chain_workspace_size(_patterns(ps), len(ps) if n is None else n, int(batch),
                                        int(dtype), int(flags), ctypes.byref(out))
    if not check:
        return st, out.value
    _raise(st, "ks_chain_workspace_size", True)
    return out.value


def ks_chain_matmul(ps: Sequence, Ws: Sequence, X, Y, batch: int, dtype: int, ws=None,
                    ws_bytes: int = 0, flags: int = CHAIN_AUTO, stream=None,
                    n: Optional[int] = None, check: bool = True) -> int:
    wp = (ctypes.c_void_p * max(len(Ws), 1))(*[_ptr(w) for w in Ws])
    st = load().ks_chain_matmul(_patterns(ps), len(ps) if n is None else n, wp, _ptr(X), _ptr(Y),
                                int(batch), int(dtype), _ptr(ws), int(ws_bytes), int(flags),
                                _stream(stream, Y, X))
    return _raise(st, "ks_chain_matmul", check)


def ks_chain_plan(ps: Sequence, batch: int, dtype: int, flags: int = CHAIN_AUTO) -> list:
    """Group lengths of a chain's launches (1 = single factor, 2 = fused pair or a
    run of two, more = a row-resident run)."""
    cap = max(len(ps), 1)
    lens = (ctypes.c_int * cap)()
    ng = ctypes.c_int(0)
    _raise(load().ks_chain_plan(_patterns(ps), len(ps), int(batch), int(dtype), int(flags), lens, cap,
                                ctypes.byref(ng)), "ks_chain_plan", True)
    return [lens[i] for i in range(ng.value)]


def ks_chain_groups(ps: Sequence, batch: int, dtype: int, flags: int = CHAIN_AUTO) -> list:
    """Factor indices of each launch group, e.g. [[0, 1], [2], [3]]."""
    out, k = [], 0
    for ln in ks_chain_plan(ps, batch, dtype, flags):
        out.append(list(range(k, k + ln)))
        k += ln
    return out


def ks_pair_closure(f, g) -> dict:
    """The closure rule for running factor f then g in one pass (ks.h)."""
    out = ks_closure_t()
    _raise(load().ks_pair_closure(_pattern(f), _pattern(g), ctypes.byref(out)), "ks_pair_closure", True)
    return {name: int(getattr(out, name)) for name, _ in ks_closure_t._fields_ if name != "reserved"}


def ks_chain_describe(ps: Sequence, batch: int, dtype: int, flags: int = CHAIN_AUTO) -> str:
    """The kernel of each launch group, "[first..last] description; ..."."""
    buf = ctypes.create_string_buffer(4096)
    _raise(load().ks_chain_describe(_patterns(ps), len(ps), int(batch), int(dtype), int(flags), buf, 4096),
           "ks_chain_describe", True)
    return buf.value.decode()


def ks_plan_describe(p, batch: int, dtype: int) -> str:
    buf = ctypes.create_string_buffer(512)
    _raise(load().ks_plan_describe(_pattern(p), int(batch), int(dtype), buf, 512), "ks_plan_describe", True)
    return buf.value.decode()


# ---------------------------------------------------------------- conveniences

def dtype_code(x_dtype, w_dtype) -> int:
    import torch
    if x_dtype == torch.float32 and w_dtype == torch.float32:
        return DTYPE_F32
    if x_dtype == torch.bfloat16 and w_dtype == torch.bfloat16:
        return DTYPE_BF16
    if x_dtype == torch.float32 and w_dtype == torch.bfloat16:
        return DTYPE_BF16W
    raise TypeError("unsupported dtypes X=%s W=%s" % (x_dtype, w_dtype))


def _check_tensor(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def matmul(X, W, pattern, out=None, kernel="auto", stream=None):
    """Y = X W^T for one KS factor; X is (batch, a*c*d), W is (a, d, b, c)."""
    import torch
    a, b, c, d = (int(v) for v in pattern)
    _check_tensor(X, "X")
    _check_tensor(W, "W")
    if X.dim() != 2 or X.shape[1] != a * c * d:
        raise ValueError("X must be (batch, a*c*d) = (*, %d)" % (a * c * d))
    if W.numel() != a * b * c * d:
        raise ValueError("W must hold a*b*c*d = %d values" % (a * b * c * d))
    batch = X.shape[0]
    if out is None:
        out = torch.empty((batch, a * b * d), dtype=torch.float32, device=X.device)
    ks_matmul_ex((a, b, c, d), W, X, out, batch, dtype_code(X.dtype, W.dtype), stream, kernel=kernel)
    return out


def chain_matmul(X, Ws, patterns, out=None, fuse=True, stream=None):
    """Apply the factors in order (factor 0 first); returns fp32 Y."""
    import torch
    _check_tensor(X, "X")
    for i, w in enumerate(Ws):
        _check_tensor(w, "W[%d]" % i)
    dt = dtype_code(X.dtype, Ws[0].dtype)
    batch = X.shape[0]
    last = patterns[-1]
    if out is None:
        out = torch.empty((batch, int(last[0]) * int(last[1]) * int(last[3])),
                          dtype=torch.float32, device=X.device)
    flags = CHAIN_AUTO if fuse else CHAIN_NO_FUSE
    nbytes = ks_chain_workspace_size(patterns, batch, dt, flags)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=X.device) if nbytes else None
    ks_chain_matmul(patterns, Ws, X, out, batch, dt, ws, nbytes, flags, stream)
    return out


def matmul_dx(dY, W, pattern, out=None, stream=None):
    """dX = dY W for one KS factor (the gradient of matmul with respect to X)."""
    import torch
    a, b, c, d = (int(v) for v in pattern)
    _check_tensor(dY, "dY")
    _check_tensor(W, "W")
    if dY.dim() != 2 or dY.shape[1] != a * b * d:
        raise ValueError("dY must be (batch, a*b*d) = (*, %d)" % (a * b * d))
    batch = dY.shape[0]
    dt = dtype_code(dY.dtype, W.dtype)
    if out is None:
        out = torch.empty((batch, a * c * d), dtype=torch.float32, device=dY.device)
    nbytes = ks_matmul_dx_workspace_size((a, b, c, d), dt)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dY.device)
    ks_matmul_dx((a, b, c, d), W, dY, out, batch, dt, ws, nbytes, stream)
    return out


def matmul_dw(dY, X, pattern, out=None, stream=None):
    """dK (shape (a, d, b, c), fp32): the gradient of matmul with respect to W."""
    import torch
    a, b, c, d = (int(v) for v in pattern)
    _check_tensor(dY, "dY")
    _check_tensor(X, "X")
    if dY.dtype != torch.float32:
        raise TypeError("dY must be fp32")
    if X.dim() != 2 or X.shape[1] != a * c * d or dY.shape != (X.shape[0], a * b * d):
        raise ValueError("X must be (batch, a*c*d) and dY (batch, a*b*d)")
    batch = X.shape[0]
    dt = DTYPE_BF16 if X.dtype == torch.bfloat16 else DTYPE_F32
    if out is None:
        out = torch.empty((a, d, b, c), dtype=torch.float32, device=X.device)
    nbytes = ks_matmul_dw_workspace_size((a, b, c, d), batch, dt)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=X.device) if nbytes else None
    ks_matmul_dw((a, b, c, d), dY, X, out, batch, dt, ws, nbytes, stream)
    return out

