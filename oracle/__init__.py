"""CPU oracle of the Q8_0 projection (ctypes over ``libq8ref.so``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only users.  The GPU library never
imports or calls it, and it never imports the GPU library.

Mode numbers follow the lane's ``activations`` knob (codegen_cuda::lane page,
description): 0 = f32 activations with f64 sums, 1 = one-word int8,
2 = two-word int8.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8ref.c")
# Q8REF_LIB names another build of the same source (the tests' sanitizer runs).
_BUILT = os.path.join(_HERE, "libq8ref.so")
_LIB_PATH = os.environ.get("Q8REF_LIB") or _BUILT
_lib = None

MODE = {"f32": 0, "i8": 1, "i8x2": 2}
BLOCK = 32
BLOCK_BYTES = 34

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int


def build() -> str:
    """Compile ``libq8ref.so`` (always recompiles).  Plain -O2, contraction off,
    no fast-math."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-o", _BUILT, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _BUILT


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        sig = {
            "q8ref_f16_bits": (ctypes.c_uint16, [ctypes.c_float]),
            "q8ref_f16_value": (ctypes.c_float, [ctypes.c_uint16]),
            "q8ref_f16_bits_array": (None, [_P, _I64, _P]),
            "q8ref_rha_array": (None, [_P, _I64, _P]),
            "q8ref_quantize_weights": (_I, [_P, _I64, _I64, _P]),
            "q8ref_dequantize_weights": (_I, [_P, _I64, _I64, _P]),
            "q8ref_quantize_act": (_I, [_I, _P, _I64, _I64, _P, _P, _P]),
            "q8ref_block_sums": (_I, [_I, _P, _I64, _I64, _I64, _P, _P, _P]),
            "q8ref_project": (_I, [_I, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
            "q8ref_project_at": (_I, [_I, _P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _I64, _P, _P,
                                      _P, _P]),
            "q8ref_dense_matvec": (None, [_P, _I64, _I64, _I64, _P, _P]),
            "q8ref_threads": (_I, []),
            "q8ref_set_threads": (None, [_I]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().q8ref_threads())


def set_threads(n: int) -> None:
    """Use n threads in the oracle's OpenMP loops from now on."""
    _load().q8ref_set_threads(int(n))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _mode(mode) -> int:
    return MODE[mode] if isinstance(mode, str) else int(mode)


def f16_bits(x) -> np.ndarray:
    """f32 -> binary16 bit patterns (round to nearest even), elementwise."""
    x = _c(np.atleast_1d(x), np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().q8ref_f16_bits_array(_ptr(x), x.size, _ptr(out))
    return out


def f16_value(h: int) -> float:
    return float(_load().q8ref_f16_value(int(h)))


def rha(x) -> np.ndarray:
    """Round half away from zero, elementwise on f32."""
    x = _c(np.atleast_1d(x), np.float32)
    out = np.empty_like(x)
    _load().q8ref_rha_array(_ptr(x), x.size, _ptr(out))
    return out


def quantize_weights(w) -> np.ndarray:
    """f32 [n][k] -> Q8_0 blocks, uint8 [n][k/32*34]."""
    w = _c(w, np.float32)
    n, k = w.shape
    out = np.empty((n, k // BLOCK * BLOCK_BYTES), dtype=np.uint8)
    if _load().q8ref_quantize_weights(_ptr(w), n, k, _ptr(out)) != 0:
        raise ValueError("k must be a multiple of 32")
    return out


def dequantize_weights(blocks, n: int, k: int) -> np.ndarray:
    blocks = _c(blocks, np.uint8)
    out = np.empty((n, k), dtype=np.float64)
    if _load().q8ref_dequantize_weights(_ptr(blocks), n, k, _ptr(out)) != 0:
        raise ValueError("k must be a multiple of 32")
    return out


def split_blocks(blocks, n: int, k: int):
    """(scale bit patterns uint16 [n][k/32], quants int8 [n][k]) of a block array."""
    b = _c(blocks, np.uint8).reshape(n, k // BLOCK, BLOCK_BYTES)
    scales = (b[:, :, 0].astype(np.uint16) | (b[:, :, 1].astype(np.uint16) << 8))
    quants = b[:, :, 2:].view(np.int8).reshape(n, k)
    return scales, quants


def quantize_act(mode, x):
    """f32 [rows][k] -> (hi int8 [rows][k], lo int8 [rows][k] or None, scale f32 [rows][k/32])."""
    m = _mode(mode)
    x = _c(np.atleast_2d(x), np.float32)
    rows, k = x.shape
    hi = np.empty((rows, k), dtype=np.int8)
    lo = np.empty((rows, k), dtype=np.int8) if m == 2 else None
    scale = np.empty((rows, k // BLOCK), dtype=np.float32)
    if _load().q8ref_quantize_act(m, _ptr(x), rows, k, _ptr(hi), _ptr(lo), _ptr(scale)) != 0:
        raise ValueError("bad mode or k")
    return hi, lo, scale


def block_sums(mode, blocks, n: int, k: int, hi, lo=None) -> np.ndarray:
    """int32 [rows][n][k/32][words] exact block dot products."""
    m = _mode(mode)
    hi = _c(np.atleast_2d(hi), np.int8)
    lo = _c(None if lo is None else np.atleast_2d(lo), np.int8)
    rows = hi.shape[0]
    words = 2 if m == 2 else 1
    out = np.empty((rows, n, k // BLOCK, words), dtype=np.int32)
    blocks = _c(blocks, np.uint8)
    if _load().q8ref_block_sums(m, _ptr(blocks), n, k, rows, _ptr(hi), _ptr(lo), _ptr(out)) != 0:
        raise ValueError("bad mode or k")
    return out


def project(mode, blocks, n: int, k: int, rows: int, hi=None, lo=None, scale=None, x=None,
            residual=None):
    """All outputs in f64: (y [rows][n], A [rows][n])."""
    m = _mode(mode)
    args = [_c(v, t) for v, t in ((hi, np.int8), (lo, np.int8), (scale, np.float32),
                                   (x, np.float32), (residual, np.float32))]
    y = np.empty((rows, n), dtype=np.float64)
    a = np.empty((rows, n), dtype=np.float64)
    blocks = _c(blocks, np.uint8)
    rc = _load().q8ref_project(m, _ptr(blocks), n, k, rows, *[_ptr(v) for v in args], _ptr(y), _ptr(a))
    if rc != 0:
        raise ValueError("bad mode or k")
    return y, a


def project_at(mode, blocks, n: int, k: int, rows: int, r_idx, n_idx, hi=None, lo=None,
               scale=None, x=None, residual=None):
    """Outputs at the (r_idx[i], n_idx[i]) pairs only, in f64: (y, A)."""
    m = _mode(mode)
    args = [_c(v, t) for v, t in ((hi, np.int8), (lo, np.int8), (scale, np.float32),
                                   (x, np.float32), (residual, np.float32))]
    r_idx = _c(r_idx, np.int64)
    n_idx = _c(n_idx, np.int64)
    y = np.empty(r_idx.size, dtype=np.float64)
    a = np.empty(r_idx.size, dtype=np.float64)
    blocks = _c(blocks, np.uint8)
    rc = _load().q8ref_project_at(m, _ptr(blocks), n, k, rows, *[_ptr(v) for v in args], r_idx.size,
                                  _ptr(r_idx), _ptr(n_idx), _ptr(y), _ptr(a))
    if rc != 0:
        raise ValueError("bad mode or k")
    return y, a


def dense_matvec(wd, v) -> np.ndarray:
    """Brute force: y[r][n] = sum_c wd[n][c] * v[r][c] in f64 by a direct loop."""
    wd = _c(wd, np.float64)
    v = _c(np.atleast_2d(v), np.float64)
    n, k = wd.shape
    rows = v.shape[0]
    y = np.empty((rows, n), dtype=np.float64)
    _load().q8ref_dense_matvec(_ptr(wd), n, k, rows, _ptr(v), _ptr(y))
    return y
