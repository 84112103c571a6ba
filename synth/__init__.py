"""Seeded synthetic inputs shared by the oracle's tests and the GPU library's tests
and benchmark.

Only random numbers live here (SplitMix64 + Box-Muller in C, see ``synth.c``);
none of the projection's arithmetic does.  Every array is a pure function of its
seed, so the CPU and GPU sides always see the same bytes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
# SYNTH_LIB names another build of the same source (the tests' sanitizer runs).
_BUILT = os.path.join(_HERE, "libsynth.so")
_LIB_PATH = os.environ.get("SYNTH_LIB") or _BUILT
_lib = None


def build() -> str:
    """Compile ``libsynth.so`` next to its source (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-o", _BUILT, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _BUILT


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_splitmix64_at.restype = ctypes.c_uint64
        lib.synth_splitmix64_at.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_normal_f32.restype = None
        lib.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_double, ctypes.c_void_p]
        lib.synth_pick.restype = ctypes.c_int
        lib.synth_pick.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_scale_rows.restype = None
        lib.synth_scale_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_float]
        lib.synth_scale_cols.restype = None
        lib.synth_scale_cols.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_float]
        _lib = lib
    return _lib


def splitmix64(seed: int, i: int) -> int:
    """Output ``i`` (0-based) of the SplitMix64 stream of ``seed``."""
    return int(_load().synth_splitmix64_at(seed & (2**64 - 1), i))


def normal(seed: int, shape, sigma: float = 1.0, offset: int = 0) -> np.ndarray:
    """float32 array of ``shape`` filled row-major from elements
    ``[offset, offset + size)`` of the normal stream of ``seed``, times ``sigma``."""
    shape = tuple(int(s) for s in (shape if isinstance(shape, (tuple, list)) else (shape,)))
    out = np.empty(shape, dtype=np.float32)
    if out.size:
        _load().synth_normal_f32(seed, int(offset), out.size, float(sigma), out.ctypes.data)
    return out


def pick(seed: int, n: int, count: int) -> np.ndarray:
    """``count`` distinct indices of ``0..n-1`` (partial Fisher-Yates on ``seed``)."""
    out = np.empty(int(count), dtype=np.int64)
    if count:
        rc = _load().synth_pick(seed, int(n), int(count), out.ctypes.data)
        if rc != 0:
            raise ValueError(f"cannot pick {count} of {n}")
    return out


def outlier_count(n: int, frac: float) -> int:
    """Number of outlier rows/channels: ``frac * n`` rounded to nearest."""
    return int(np.floor(frac * n + 0.5))


def weights(n: int, k: int, seed: int, sigma: float = 0.02,
            outlier_frac: float = 0.0, outlier_scale: float = 8.0) -> np.ndarray:
    """f32 weight matrix [n][k] ~ N(0, sigma^2); optionally a fraction of whole rows
    (picked on stream ``seed + 1000``) multiplied by ``outlier_scale``."""
    w = normal(seed, (n, k), sigma)
    cnt = outlier_count(n, outlier_frac)
    if cnt:
        rows = pick(seed + 1000, n, cnt)
        _load().synth_scale_rows(w.ctypes.data, k, rows.ctypes.data, cnt, float(outlier_scale))
    return w


def activations(rows: int, k: int, seed: int | None = None, row_seeds=None, sigma: float = 1.0,
                outlier_frac: float = 0.0, outlier_scale: float = 20.0) -> np.ndarray:
    """f32 activation stack [rows][k] ~ N(0, sigma^2).

    Either one stream for the whole stack (``seed``) or one independent stream per
    row (``row_seeds``).  Optionally a fraction of channels (columns, picked on
    stream ``seed + 1000``, or the first row seed + 1000) is multiplied by
    ``outlier_scale`` in every row."""
    if row_seeds is not None:
        row_seeds = list(row_seeds)
        assert len(row_seeds) == rows
        x = np.stack([normal(s, k, sigma) for s in row_seeds]) if rows else np.empty((0, k), np.float32)
        base = row_seeds[0] if rows else 0
    else:
        x = normal(seed, (rows, k), sigma)
        base = seed
    cnt = outlier_count(k, outlier_frac)
    if cnt and rows:
        chans = pick(base + 1000, k, cnt)
        x = np.ascontiguousarray(x)
        _load().synth_scale_cols(x.ctypes.data, rows, k, chans.ctypes.data, cnt, float(outlier_scale))
    return x
