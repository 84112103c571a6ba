"""Mistakes planted in a copy of the oracle must each fail a pin.

Each mutant is the oracle's C source with one plausible slip (a dropped term, a
wrong sign or index, the wrong rounding, the wrong scale), compiled to a
temporary library on the CPU.  The pins below (hand-worked blocks, library
routines, brute force) are run against it; at least one must fail.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth

from test_oracle import _error_scale_numpy, block_from, read_golden

SRC = os.path.join(os.path.dirname(oracle.__file__), "q8ref.c")

MUTANTS = {
    "half_even_rounding": ("static float rha(float v) { return roundf(v); }",
                           "static float rha(float v) { return rintf(v); }"),
    "weights_divided_by_f32_scale": ("clamp127(rha(src[j] / dq))", "clamp127(rha(src[j] / d32))"),
    "two_word_lo_dropped": ("(double)sh + (double)sl / 128.0 : (double)sh",
                            "(double)sh : (double)sh"),
    "two_word_lo_sign": ("(double)sh + (double)sl / 128.0", "(double)sh - (double)sl / 128.0"),
    "lo_scale_128_missing": ("rha((resid * 128.0f) / s)", "rha(resid / s)"),
    "block_sum_wrong_row": ("sh += (int32_t)q[j] * (int32_t)hi[r * k + b * Q8_BLOCK + j];",
                            "sh += (int32_t)q[j] * (int32_t)hi[b * Q8_BLOCK + j];"),
    "act_scale_wrong_block": ("double s = (double)scale[r * nb + b];",
                              "double s = (double)scale[r * nb + (b + 1) % nb];"),
    "f16_truncates": ("double m = rint(a / quantum);", "double m = floor(a / quantum);"),
    "residual_dropped": ("        y += res;\n", "        (void)res;\n"),
    "f32_mode_weight_scale_dropped": ("            term = d * p;", "            term = p;"),
    "error_scale_doubled": ("        a += fabs(term);\n", "        a += 2.0 * fabs(term);\n"),
    "error_scale_signed": ("        a += fabs(term);\n", "        a += term;\n"),
    "error_scale_residual_twice": ("        a += fabs(res);\n", "        a += 2.0 * fabs(res);\n"),
    "amax_signed": ("if (fabsf(src[j]) > amax) amax = fabsf(src[j]);\n            float s",
                    "if (src[j] > amax) amax = src[j];\n            float s"),
}


def _pins():
    """Run the pins against whatever library oracle._lib holds; return failures."""
    failures = []

    def check(name, cond):
        if not cond:
            failures.append(name)

    ga, gb = read_golden("act_block_a.txt"), read_golden("act_block_b.txt")
    gw, gd = read_golden("weight_block_w1.txt"), read_golden("dot_w1_a.txt")
    for tag, g in (("A", ga), ("B", gb)):
        hi, lo, s = oracle.quantize_act("i8x2", block_from(g["x"]))
        check(f"golden act {tag}", hi[0].tolist() == [int(v) for v in g["hi"]]
              and lo[0].tolist() == [int(v) for v in g["lo"]] and s[0, 0] == float(g["scale"][0]))
    w1 = (np.array([float(v) for v in gw["k_over_128"]]) / 128.0).astype(np.float32)[None, :]
    blocks = oracle.quantize_weights(w1)
    check("golden weight", blocks[0].tolist() == [int(v, 16) for v in gw["block_bytes"]])
    hi, lo, s = oracle.quantize_act("i8x2", block_from(ga["x"]))
    y2, _ = oracle.project("i8x2", blocks, 1, 32, 1, hi=hi, lo=lo, scale=s,
                           residual=np.array([[0.5]], np.float32))
    y0, _ = oracle.project("f32", blocks, 1, 32, 1, x=block_from(ga["x"]))
    check("golden dot", y2[0, 0] == float(gd["y_i8x2"][0]) + 0.5 and y0[0, 0] == float(gd["y_f32"][0]))

    x16 = np.array([1.0009765625 + 2.0 ** -11, 3.0e-3, 1.0 / 127, 0.04 / 127], np.float32)
    check("f16 vs numpy", np.array_equal(oracle.f16_bits(x16), x16.astype(np.float16).view(np.uint16)))

    n, k, rows = 17, 128, 3
    w = synth.weights(n, k, seed=12, outlier_frac=0.1)
    x = synth.activations(rows, k, seed=62, outlier_frac=0.05)
    b = oracle.quantize_weights(w)
    wd = oracle.dequantize_weights(b, n, k)
    scales, _ = oracle.split_blocks(b, n, k)
    dqe = np.repeat(scales.view(np.float16).astype(np.float64), 32, axis=1)
    check("weight half step", (np.abs(wd - w.astype(np.float64)) <= dqe * (0.5 + 2.0 ** -16)).all())
    for mode in ("i8", "i8x2"):
        hi, lo, s = oracle.quantize_act(mode, x)
        se = np.repeat(s.astype(np.float64), 32, axis=1)
        v = se * hi if mode == "i8" else se * (hi + lo / 128.0)
        y, a = oracle.project(mode, b, n, k, rows, hi=hi, lo=lo, scale=s)
        check(f"brute {mode}", (np.abs(y - v @ wd.T) <= 1e-12 * a).all())
        sums = oracle.block_sums(mode, b, n, k, hi, lo)
        _, q = oracle.split_blocks(b, n, k)
        ref = np.einsum("nbj,rbj->rnb", q.reshape(n, k // 32, 32).astype(np.int64),
                        hi.reshape(rows, k // 32, 32).astype(np.int64))
        check(f"sums {mode}", np.array_equal(sums[..., 0], ref))
        err = np.abs(v - x.astype(np.float64))
        step = 0.5 if mode == "i8" else 1.0 / 256
        check(f"act bound {mode}", (err <= se * (step + 2.0 ** -16)).all())
    y, a = oracle.project("f32", b, n, k, rows, x=x)
    check("brute f32", (np.abs(y - x.astype(np.float64) @ wd.T) <= 1e-12 * a).all())
    res = synth.normal(63, (rows, n))
    for mode in ("f32", "i8", "i8x2"):
        if mode == "f32":
            _, a = oracle.project(mode, b, n, k, rows, x=x, residual=res)
        else:
            hi, lo, s = oracle.quantize_act(mode, x)
            _, a = oracle.project(mode, b, n, k, rows, hi=hi, lo=lo, scale=s, residual=res)
        check(f"error scale {mode}", np.allclose(a, _error_scale_numpy(mode, b, n, k, x, res), rtol=1e-12, atol=0.0))
    return failures


def test_pins_pass_on_the_oracle():
    assert _pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    lib_path = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                    "-o", str(lib_path), str(mutant), "-lm"], check=True)
    saved = oracle._load()
    try:
        lib = ctypes.CDLL(str(lib_path))
        for fname in ("q8ref_f16_bits", "q8ref_f16_value", "q8ref_f16_bits_array", "q8ref_rha_array",
                      "q8ref_quantize_weights", "q8ref_dequantize_weights", "q8ref_quantize_act",
                      "q8ref_block_sums", "q8ref_project", "q8ref_project_at", "q8ref_dense_matvec"):
            fn, ref = getattr(lib, fname), getattr(saved, fname)
            fn.restype, fn.argtypes = ref.restype, ref.argtypes
        oracle._lib = lib
        failures = _pins()
    finally:
        oracle._lib = saved
    assert failures, f"mutant {name} passed every pin"
