"""Shared helpers of the GPU parity tests: the output gate, and cached inputs.

The gate for an f32 output y against the oracle's f64 result R (with error scale
A = sum of |block terms| + |residual|):   |y - R| <= 1e-5 |R| + 2^-40 A.
The library sums block terms in f64 and rounds once, so |y - R| is one f32
rounding (2^-24 |R|) plus f64 summation-order differences (< 2 * 448 * 2^-53 A
at the largest block count); 2^-40 A covers the latter with a wide margin.

The gate also asserts that y is at most one f32 step from fl32(R) wherever that
follows from the f64 sums: if the library's f64 total T and R differ by at most
2^-40 A <= u/4, with u the f32 spacing of the binade of |R|, then fl32(T) and
fl32(R) are equal or adjacent.  Outputs that cancel to near zero (A large
against |R|) are held to the gate alone.
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


def ulp_distance(y: np.ndarray, r: np.ndarray) -> np.ndarray:
    """f32 steps between y and fl32(r) (same-sign values: bit-pattern distance)."""
    r32 = np.asarray(r, dtype=np.float64).astype(np.float32)
    yb = np.ascontiguousarray(y, dtype=np.float32).view(np.int32).astype(np.int64)
    rb = np.ascontiguousarray(r32).view(np.int32).astype(np.int64)
    return np.abs(yb - rb)


def ulp_eligible(r: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Outputs where the f64 order bound 2^-40 A is within a quarter of the f32
    spacing of R's binade."""
    _, e = np.frexp(np.abs(r))
    spacing = np.ldexp(1.0, e - 24)          # f32 spacing of [2^(e-1), 2^e)
    return (ABS_A * a <= spacing / 4) & (r != 0)


def gate(y: np.ndarray, r: np.ndarray, a: np.ndarray, what: str = ""):
    """Assert the per-element gate and the one-step bound; return (max rel err,
    max ulps vs fl32(R) over the outputs the bound covers)."""
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
    ulps = ulp_distance(y, r)
    ok = ulp_eligible(r, a)
    far = ok & (ulps > 1)
    if far.any():
        i = np.flatnonzero(far.ravel())[:5]
        raise AssertionError(
            f"{what}: {int(far.sum())} outputs more than one f32 step from fl32(R); first "
            f"{[(int(j), float(y.ravel()[j]), float(r.ravel()[j]), int(ulps.ravel()[j])) for j in i]}")
    return rel, int(ulps[ok].max()) if ok.any() else 0


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
