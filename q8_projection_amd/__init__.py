"""Python binding of libq8proj.so, the MI355X Q8_0 projection library.

Argument marshalling only: every step of the projection runs in the library's
HIP kernels.  PyTorch provides device memory and streams; output tensors are
allocated here with ``torch.empty`` when the caller passes none.  The names and
arguments mirror the C ABI in ``include/q8.h``; see there for layouts,
numerics and errors.

The library must be built (``python q8_projection_amd/build.py``); importing
this module without it, or calling a projection without a GPU, raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# Q8PROJ_LIB names another build of the same sources (the tests' host-sanitizer run).
LIB_PATH = os.environ.get("Q8PROJ_LIB") or os.path.join(_HERE, "libq8proj.so")

MODES = {"f32": 0, "i8": 1, "i8x2": 2}
STATUS = {0: "Q8_OK", 1: "Q8_E_NULL", 2: "Q8_E_SHAPE", 3: "Q8_E_ALIGN", 4: "Q8_E_MODE",
          5: "Q8_E_ALIAS", 6: "Q8_E_HIP"}
BLOCK = 32
BLOCK_BYTES = 34

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int

# Exported symbols and their C signatures (include/q8.h).
SIGNATURES = {
    "q8_quantize_weights": (_I, [_P, _I64, _I64, _P, _P]),
    "q8_quantize_act": (_I, [_I, _P, _I64, _I64, _P, _P, _P, _P]),
    "q8_matvec": (_I, [_I, _P, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "q8_matmul_rows": (_I, [_I, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "q8_matmul_rows_ws": (_I, [_I, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _I64, _P]),
    "q8_matmul_rows_workspace_bytes": (_I64, [_I, _I64, _I64, _I64]),
    "q8_matvec_argmax": (_I, [_I, _P, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "q8_argmax_workspace_bytes": (_I64, [_I64]),
    "q8_matvec_argmax_noalloc": (_I, [_I, _P, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "q8_block_sums": (_I, [_I, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "q8_status_name": (ctypes.c_char_p, [_I]),
    "q8_version": (_I, []),
}

_lib = None


class Q8Error(RuntimeError):
    """A named status other than Q8_OK returned by the library."""

    def __init__(self, fn: str, status: int):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{fn}: {self.name}")


def lib() -> ctypes.CDLL:
    """The loaded ``libq8proj.so``; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with q8_projection_amd/build.py")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_name(status: int) -> str:
    return lib().q8_status_name(int(status)).decode()


def version() -> int:
    return int(lib().q8_version())


def _mode(mode) -> int:
    return MODES[mode] if isinstance(mode, str) else int(mode)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, status: int):
    if status != 0:
        raise Q8Error(fn, status)


def _want(t, name: str, dtype, numel: int, optional: bool = False):
    """Raise ValueError unless t is a contiguous device tensor of `dtype` with at
    least `numel` elements (or None where the argument is optional): the library
    reads or writes that many elements from the pointer it is given."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, {numel} needed")


def _want_weights(w, n: int, k: int):
    _want(w, "w", torch.uint8, n * (k // BLOCK) * BLOCK_BYTES)


def _want_stack(m: int, rows: int, k: int, hi, lo, scale, x):
    """The activation arguments of a projection: the quantized stack (hi, lo,
    scale) or, in the f32 mode or to quantize inside the call, x."""
    if m == 0 or (hi is None and lo is None and scale is None):
        _want(x, "x", torch.float32, rows * k)
        return
    _want(hi, "hi", torch.int8, rows * k)
    _want(lo, "lo", torch.int8, rows * k, optional=m != 2)
    _want(scale, "scale", torch.float32, rows * (k // BLOCK))


def _device_of(*ts):
    for t in ts:
        if t is not None:
            return t.device
    raise ValueError("no tensor argument")


def quantize_weights(w: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Q8_0 blocks (uint8 [n][k/32*34]) of an f32 [n][k] matrix."""
    n, k = w.shape
    _want(w, "w", torch.float32, n * k)
    if out is None:
        out = torch.empty((n, (k // BLOCK) * BLOCK_BYTES), dtype=torch.uint8, device=w.device)
    _want(out, "out", torch.uint8, n * (k // BLOCK) * BLOCK_BYTES)
    _check("q8_quantize_weights", lib().q8_quantize_weights(_ptr(w), n, k, _ptr(out), _stream(stream)))
    return out


def quantize_act(mode, x: torch.Tensor, hi=None, lo=None, scale=None, stream=None):
    """(hi int8 [rows][k], lo int8 [rows][k] or None, scale f32 [rows][k/32]) of an
    f32 [rows][k] stack (a 1-D x is one row)."""
    m = _mode(mode)
    x2 = x if x.dim() == 2 else x.view(1, -1)
    rows, k = x2.shape
    _want(x2, "x", torch.float32, rows * k)
    dev = x.device
    if hi is None:
        hi = torch.empty((rows, k), dtype=torch.int8, device=dev)
    if m == 2 and lo is None:
        lo = torch.empty((rows, k), dtype=torch.int8, device=dev)
    if scale is None:
        scale = torch.empty((rows, k // BLOCK), dtype=torch.float32, device=dev)
    _want(hi, "hi", torch.int8, rows * k)
    _want(lo, "lo", torch.int8, rows * k, optional=m != 2)
    _want(scale, "scale", torch.float32, rows * (k // BLOCK))
    _check("q8_quantize_act", lib().q8_quantize_act(m, _ptr(x2), rows, k, _ptr(hi),
                                                    _ptr(lo if m == 2 else None), _ptr(scale),
                                                    _stream(stream)))
    return hi, (lo if m == 2 else None), scale


def matmul_rows(mode, w: torch.Tensor, n: int, k: int, hi=None, lo=None, scale=None, x=None,
                residual=None, out=None, rows: int | None = None, stream=None) -> torch.Tensor:
    """Y [rows][n] = X W^T (+ residual) over a stack of activation rows.  In an
    integer mode, x alone (hi, lo, scale None) is quantized inside the call, for
    stacks of at most 8 rows."""
    m = _mode(mode)
    src = x if (m == 0 or hi is None) else hi
    if rows is None:
        rows = 1 if src is None or src.dim() == 1 else src.shape[0]
    if out is None:
        out = torch.empty((rows, n), dtype=torch.float32, device=_device_of(w, src))
    _want_weights(w, n, k)
    _want_stack(m, rows, k, hi, lo, scale, x)
    _want(residual, "residual", torch.float32, rows * n, optional=True)
    _want(out, "out", torch.float32, rows * n)
    _check("q8_matmul_rows", lib().q8_matmul_rows(m, _ptr(w), n, k, rows, _ptr(hi), _ptr(lo), _ptr(scale),
                                                  _ptr(x), _ptr(residual), _ptr(out), _stream(stream)))
    return out


def matmul_rows_workspace_bytes(mode, n: int, k: int, rows: int) -> int:
    """Bytes of the matmul_rows_ws workspace for this call (0: it does not split K)."""
    return int(lib().q8_matmul_rows_workspace_bytes(_mode(mode), n, k, rows))


def matmul_rows_ws(mode, w: torch.Tensor, n: int, k: int, hi=None, lo=None, scale=None, x=None,
                   residual=None, out=None, workspace=None, rows: int | None = None, stream=None) -> torch.Tensor:
    """matmul_rows with K split across workgroups for integer stacks on short
    matrices (q8_matmul_rows_ws).  The workspace (uint8, at least
    matmul_rows_workspace_bytes) must start zero-filled; each call leaves its
    counters at zero, so a caller may keep one per stream and pass it every
    time.  None allocates a zero-filled one for this call."""
    m = _mode(mode)
    src = x if (m == 0 or hi is None) else hi
    if rows is None:
        rows = 1 if src is None or src.dim() == 1 else src.shape[0]
    dev = _device_of(w, src)
    if out is None:
        out = torch.empty((rows, n), dtype=torch.float32, device=dev)
    need = matmul_rows_workspace_bytes(mode, n, k, rows)
    if workspace is None and need > 0:
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)
    _want_weights(w, n, k)
    _want_stack(m, rows, k, hi, lo, scale, x)
    _want(residual, "residual", torch.float32, rows * n, optional=True)
    _want(out, "out", torch.float32, rows * n)
    _want(workspace, "workspace", torch.uint8, need, optional=True)
    wsb = 0 if workspace is None else workspace.numel()
    _check("q8_matmul_rows_ws", lib().q8_matmul_rows_ws(m, _ptr(w), n, k, rows, _ptr(hi), _ptr(lo), _ptr(scale),
                                                        _ptr(x), _ptr(residual), _ptr(out), _ptr(workspace), wsb,
                                                        _stream(stream)))
    return out


def matvec(mode, w: torch.Tensor, n: int, k: int, hi=None, lo=None, scale=None, x=None,
           residual=None, out=None, stream=None) -> torch.Tensor:
    """y [n] = W x (+ residual) for one activation row."""
    m = _mode(mode)
    if out is None:
        out = torch.empty((n,), dtype=torch.float32, device=_device_of(w, hi, x))
    _want_weights(w, n, k)
    _want_stack(m, 1, k, hi, lo, scale, x)
    _want(residual, "residual", torch.float32, n, optional=True)
    _want(out, "out", torch.float32, n)
    _check("q8_matvec", lib().q8_matvec(m, _ptr(w), n, k, _ptr(hi), _ptr(lo), _ptr(scale), _ptr(x),
                                        _ptr(residual), _ptr(out), _stream(stream)))
    return out


def argmax_workspace_bytes(n: int) -> int:
    """Bytes of the matvec_argmax workspace for n weight rows."""
    return int(lib().q8_argmax_workspace_bytes(n))


def matvec_argmax(mode, w: torch.Tensor, n: int, k: int, hi=None, lo=None, scale=None, x=None,
                  residual=None, out=None, idx=None, workspace=None, stream=None):
    """(y [n], idx) with idx = argmax y (lowest index among equal maxima), one launch.
    The workspace must start zero-filled; each call puts its counter (the first
    16 bytes) back to zero, so a caller may keep one per stream and pass it
    every time."""
    m = _mode(mode)
    dev = _device_of(w, hi, x)
    if out is None:
        out = torch.empty((n,), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((1,), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.zeros(max(16, argmax_workspace_bytes(n)), dtype=torch.uint8, device=dev)
    _want_weights(w, n, k)
    _want_stack(m, 1, k, hi, lo, scale, x)
    _want(residual, "residual", torch.float32, n, optional=True)
    _want(out, "out", torch.float32, n)
    _want(idx, "idx", torch.int32, 1)
    _want(workspace, "workspace", torch.uint8, argmax_workspace_bytes(n))
    _check("q8_matvec_argmax", lib().q8_matvec_argmax(m, _ptr(w), n, k, _ptr(hi), _ptr(lo), _ptr(scale), _ptr(x),
                                                      _ptr(residual), _ptr(out), _ptr(idx), _ptr(workspace),
                                                      _stream(stream)))
    return out, idx


def matvec_argmax_noalloc(mode, w: torch.Tensor, n: int, k: int, hi=None, lo=None, scale=None, x=None,
                          residual=None, out=None, idx=None, stream=None):
    """matvec_argmax with the library's own fixed workspace (q8_matvec_argmax_noalloc):
    the call itself allocates nothing when out and idx are given.  Calls that
    overlap on one GPU race."""
    m = _mode(mode)
    dev = _device_of(w, hi, x)
    if out is None:
        out = torch.empty((n,), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((1,), dtype=torch.int32, device=dev)
    _want_weights(w, n, k)
    _want_stack(m, 1, k, hi, lo, scale, x)
    _want(residual, "residual", torch.float32, n, optional=True)
    _want(out, "out", torch.float32, n)
    _want(idx, "idx", torch.int32, 1)
    _check("q8_matvec_argmax_noalloc",
           lib().q8_matvec_argmax_noalloc(m, _ptr(w), n, k, _ptr(hi), _ptr(lo), _ptr(scale), _ptr(x),
                                          _ptr(residual), _ptr(out), _ptr(idx), _stream(stream)))
    return out, idx


def block_sums(mode, w: torch.Tensor, n: int, k: int, hi, lo=None, out=None, rows: int | None = None,
               stream=None) -> torch.Tensor:
    """Exact int32 block dot products [rows][n][k/32][words]."""
    m = _mode(mode)
    if rows is None:
        rows = 1 if hi.dim() == 1 else hi.shape[0]
    words = 2 if m == 2 else 1
    if out is None:
        out = torch.empty((rows, n, k // BLOCK, words), dtype=torch.int32, device=hi.device)
    _want_weights(w, n, k)
    _want(hi, "hi", torch.int8, rows * k)
    _want(lo, "lo", torch.int8, rows * k, optional=m != 2)
    _want(out, "out", torch.int32, rows * n * (k // BLOCK) * words)
    _check("q8_block_sums", lib().q8_block_sums(m, _ptr(w), n, k, rows, _ptr(hi), _ptr(lo), _ptr(out),
                                                _stream(stream)))
    return out
