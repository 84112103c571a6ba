"""Shared helpers of the GPU parity tests: the output gate, and cached inputs.

The gate for an f32 output y against the oracle's f64 result R (with error scale
A = sum of |block terms| + |residual|):   |y - R| <= 1e-5 |R| + 2^-40 A.
The library sums block terms in f64 and rounds once, so |y - R| is one f32
rounding (2^-24 |R|) plus f64 summation-order differences (< 448 * 2^-53 A at the
largest block count); 2^-40 A covers the latter with a wide margin.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

REL_TOL = 1e-5
ABS_A = 2.0 ** -40

_cache: dict = {}


def say(*msg):
    print("[case]", *msg, file=sys.stderr, flush=True)


def gate(y: np.ndarray, r: np.ndarray, a: np.ndarray, what: str = ""):
    """Assert the per-element gate; return (max rel err, max ulps vs fl32(R))."""
    y64 = y.astype(np.float64)
    err = np.abs(y64 - r)
    bound = REL_TOL * np.abs(r) + ABS_A * a
    bad = err > bound
    if bad.any():
        i = np.flatnonzero(bad.ravel())[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outputs outside the gate; first "
            f"{[(int(j), float(y.ravel()[j]), float(r.ravel()[j]), float(a.ravel()[j])) for j in i]}")
    rel = float(np.max(err / np.maximum(np.abs(r), 1e-300))) if r.size else 0.0
    r32 = r.astype(np.float32)
    ulps = np.abs(y.view(np.int32).astype(np.int64) - r32.view(np.int32).astype(np.int64))
    return rel, int(ulps.max()) if ulps.size else 0


def weights_of(call):
    key = ("w", call.n, call.k, call.w_seed, call.w_outlier_frac, call.w_outlier_scale)
    if key not in _cache:
        w = call.make_weights()
        _cache[key] = (w, oracle.quantize_weights(w))
    return _cache[key]


def acts_of(call):
    key = ("x", call.rows, call.k, call.x_seed, call.x_row_seeds, call.x_rows_total, call.last_row_only,
           call.x_outlier_frac, call.x_outlier_scale)
    if key not in _cache:
        _cache[key] = call.make_activations()
    return _cache[key]


def drop_cache():
    _cache.clear()
