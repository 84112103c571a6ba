"""Pins of the CPU oracle against things other than itself: hand-worked blocks,
library routines, invariants of the quantizers, closed-form error bounds and
brute force on tiny shapes.  CPU only.

Numerics come from the codegen_cuda::lane page, description (the `activations`
knob) and the model::author page, description (Q8_0 quants and block scales).
"""
import os

import numpy as np
import pytest

import oracle
import synth
from synth import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split(":", 1)
            out[key.strip()] = vals.split()
    return out


def block_from(vals, k=32):
    x = np.zeros((1, k), dtype=np.float32)
    x[0, :32] = np.array([float(v) for v in vals], dtype=np.float64).astype(np.float32)
    return x


# ----------------------------------------------------------------- golden blocks

@pytest.mark.parametrize("fixture", ["act_block_a.txt", "act_block_b.txt"])
def test_golden_activation_block(fixture):
    g = read_golden(fixture)
    x = block_from(g["x"])
    # the fixture's decimal strings are the exact f32 values
    for s, v in zip(g["x"], x[0]):
        assert float(s) == float(v)
    hi, lo, scale = oracle.quantize_act("i8x2", x)
    assert scale[0, 0] == np.float32(float(g["scale"][0]))
    assert hi[0].tolist() == [int(v) for v in g["hi"]]
    assert lo[0].tolist() == [int(v) for v in g["lo"]]
    hi1, lo1, scale1 = oracle.quantize_act("i8", x)
    assert lo1 is None
    assert np.array_equal(hi1, hi) and np.array_equal(scale1, scale)


def test_golden_weight_block():
    g = read_golden("weight_block_w1.txt")
    w = (np.array([float(v) for v in g["k_over_128"]]) / 128.0).astype(np.float32)[None, :]
    blocks = oracle.quantize_weights(w)
    expect = [int(v, 16) for v in g["block_bytes"]]
    assert len(expect) == 34
    assert blocks[0].tolist() == expect
    scales, quants = oracle.split_blocks(blocks, 1, 32)
    assert int(scales[0, 0]) == int(g["scale_bits"][0], 16)
    assert oracle.f16_value(0x2000) == 2.0 ** -7


def test_golden_dot():
    ga = read_golden("act_block_a.txt")
    gw = read_golden("weight_block_w1.txt")
    gd = read_golden("dot_w1_a.txt")
    x = block_from(ga["x"])
    w = (np.array([float(v) for v in gw["k_over_128"]]) / 128.0).astype(np.float32)[None, :]
    blocks = oracle.quantize_weights(w)
    hi, lo, scale = oracle.quantize_act("i8x2", x)
    sums = oracle.block_sums("i8x2", blocks, 1, 32, hi, lo)
    assert sums[0, 0, 0].tolist() == [int(gd["s_hi"][0]), int(gd["s_lo"][0])]
    sums1 = oracle.block_sums("i8", blocks, 1, 32, hi)
    assert sums1[0, 0, 0].tolist() == [int(gd["s_hi"][0])]
    y1, _ = oracle.project("i8", blocks, 1, 32, 1, hi=hi, scale=scale)
    y2, _ = oracle.project("i8x2", blocks, 1, 32, 1, hi=hi, lo=lo, scale=scale)
    y0, _ = oracle.project("f32", blocks, 1, 32, 1, x=x)
    assert y1[0, 0] == float(gd["y_i8"][0])
    assert y2[0, 0] == float(gd["y_i8x2"][0])
    assert y0[0, 0] == float(gd["y_f32"][0])
    # a residual is added in f64
    r = np.array([[0.5]], dtype=np.float32)
    y2r, a2r = oracle.project("i8x2", blocks, 1, 32, 1, hi=hi, lo=lo, scale=scale, residual=r)
    assert y2r[0, 0] == float(gd["y_i8x2"][0]) + 0.5
    assert a2r[0, 0] >= abs(y2r[0, 0])


def test_zero_blocks():
    x = np.zeros((2, 64), np.float32)
    x[1, 32:] = 1.0                       # second block of row 1 nonzero
    hi, lo, s = oracle.quantize_act("i8x2", x)
    assert s[0].tolist() == [0.0, 0.0] and s[1, 0] == 0.0
    assert not hi[0].any() and not lo[0].any() and not hi[1, :32].any()
    assert (hi[1, 32:] == 127).all() and not lo[1, 32:].any()
    w = np.zeros((1, 64), np.float32)
    blocks = oracle.quantize_weights(w)
    assert not blocks.any()


def test_tiny_values_underflow_scale():
    # block max so small that max/127 underflows to zero in f32: all quants 0
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = np.float32(2.0 ** -149)
    hi, lo, s = oracle.quantize_act("i8x2", x)
    assert s[0, 0] == 0.0 and not hi.any() and not lo.any()
    # a binary16 scale that rounds to zero gives all-zero weight quants
    w = np.zeros((1, 32), np.float32)
    w[0, 3] = np.float32(2.0 ** -40)
    blocks = oracle.quantize_weights(w)
    assert not blocks.any()


# ------------------------------------------------------------ library routines

def _f32_from_bits(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _check_f16_bits(bits):
    x = _f32_from_bits(bits)
    x = x[~np.isnan(x)]
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
        ref_neg = (-x).astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f16_bits(x), ref)
    assert np.array_equal(oracle.f16_bits(-x), ref_neg)


def test_f16_against_numpy_sweep():
    """f32 -> binary16 RNE against numpy's float16 cast: a stride-97 sweep over
    every positive f32 bit pattern (and its negation), which visits every binade,
    the subnormal range and the overflow edge, plus every pattern of the binades
    at the subnormal boundary and of a typical weight-scale binade."""
    _check_f16_bits(np.arange(0, 1 << 31, 97, dtype=np.uint64).astype(np.uint32))
    for lo_exp in (-25, -15, -14, -8, 15):
        lo_bits = int(np.array([2.0 ** lo_exp], np.float32).view(np.uint32)[0])
        _check_f16_bits(np.arange(lo_bits, lo_bits + (1 << 23), dtype=np.uint64).astype(np.uint32))


def test_f16_ties_and_edges():
    # exact ties between binary16 neighbours in every binade and in the subnormals
    vals = []
    for e in range(-24, 16):
        q = 2.0 ** (max(e, -14) - 10)
        base = 2.0 ** e
        for m in range(0, 8):
            vals.append(base + (m + 0.5) * q)
    vals += [65504.0, 65519.99, 65520.0, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -24,
             1.5 * 2.0 ** -24, 6.1035156e-05, 6.097555e-05]
    x = np.array(vals, dtype=np.float64).astype(np.float32)
    x = np.concatenate([x, -x])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f16_bits(x), ref)
    for h in [0x0001, 0x03ff, 0x0400, 0x3c00, 0x7bff, 0x8001, 0xfbff, 0x2000]:
        assert oracle.f16_value(h) == float(np.array([h], np.uint16).view(np.float16)[0])


def _rha_ref(x):
    x64 = np.asarray(x, dtype=np.float64)
    return (np.sign(x64) * np.floor(np.abs(x64) + 0.5)).astype(np.float32)


def test_round_half_away():
    special = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 0.49999997, -0.49999997, 0.0, -0.0,
                        8388607.5, 8388608.5, 16777216.0, 126.5, -126.5, 127.49999], np.float32)
    expect = np.array([1, 2, 3, -1, -2, -3, 0, 0, 0, 0, 8388608, 8388608, 16777216, 127, -127, 127],
                      np.float32)
    assert np.array_equal(oracle.rha(special), expect)
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(1 << 20) * 200).astype(np.float32)
    x = np.concatenate([x, np.round(x) + np.float32(0.5), np.round(x) - np.float32(0.5)])
    assert np.array_equal(oracle.rha(x), _rha_ref(x))


def test_block_sums_against_einsum():
    rng = np.random.default_rng(7)
    n, k, rows = 37, 256, 5
    w = synth.weights(n, k, seed=101)
    x = synth.activations(rows, k, seed=102)
    blocks = oracle.quantize_weights(w)
    hi, lo, s = oracle.quantize_act("i8x2", x)
    sums = oracle.block_sums("i8x2", blocks, n, k, hi, lo)
    _, q = oracle.split_blocks(blocks, n, k)
    qb = q.reshape(n, k // 32, 32).astype(np.int64)
    ref_hi = np.einsum("nbj,rbj->rnb", qb, hi.reshape(rows, k // 32, 32).astype(np.int64))
    ref_lo = np.einsum("nbj,rbj->rnb", qb, lo.reshape(rows, k // 32, 32).astype(np.int64))
    assert np.array_equal(sums[..., 0], ref_hi)
    assert np.array_equal(sums[..., 1], ref_lo)
    del rng


# ---------------------------------------------------------------- invariants

def _small_configs():
    """Small shapes with each workload's value distributions."""
    return [
        dict(n=64, k=1024, w=dict(seed=0), x=dict(seed=1)),
        dict(n=96, k=512, w=dict(seed=2, outlier_frac=0.05, outlier_scale=8.0),
             x=dict(seed=3, outlier_frac=0.02, outlier_scale=20.0)),
        dict(n=40, k=2048, w=dict(seed=7), x=dict(seed=9)),
    ]


@pytest.mark.parametrize("cfg", _small_configs())
def test_weight_quant_invariants(cfg):
    n, k = cfg["n"], cfg["k"]
    w = synth.weights(n, k, **cfg["w"])
    blocks = oracle.quantize_weights(w)
    scales, q = oracle.split_blocks(blocks, n, k)
    dq = scales.astype(np.uint16).view(np.float16).astype(np.float64)          # numpy decode
    dqe = np.repeat(dq, 32, axis=1)
    err = np.abs(dqe * q.astype(np.float64) - w.astype(np.float64))
    assert (err <= dqe * (0.5 + 2.0 ** -16)).all()
    # the scale is binary16(max|w|/127) and the max element maps to +-127
    amax = np.abs(w.reshape(n, k // 32, 32)).max(axis=2)
    assert np.array_equal(scales, (amax / np.float32(127)).astype(np.float32).astype(np.float16).view(np.uint16))
    qb = np.abs(q.reshape(n, k // 32, 32)).max(axis=2)
    assert (qb == 127).all()
    # idempotence: quantizing the dequantized matrix gives the same bytes
    wd = (dqe * q).astype(np.float32)
    assert np.array_equal(oracle.quantize_weights(wd), blocks)
    # sign symmetry
    bn = oracle.quantize_weights(-w)
    sn, qn = oracle.split_blocks(bn, n, k)
    assert np.array_equal(sn, scales) and np.array_equal(qn, -q)


@pytest.mark.parametrize("cfg", _small_configs())
def test_act_quant_invariants(cfg):
    k = cfg["k"]
    rows = 3
    x = synth.activations(rows, k, **cfg["x"])
    hi, lo, s = oracle.quantize_act("i8x2", x)
    se = np.repeat(s.astype(np.float64), 32, axis=1)
    x64 = x.astype(np.float64)
    assert (np.abs(se * hi - x64) <= se * (0.5 + 2.0 ** -16)).all()
    assert (np.abs(se * (hi + lo / 128.0) - x64) <= se * (1.0 / 256 + 2.0 ** -16)).all()
    assert (np.abs(lo) <= 64).all()
    amax = np.abs(x.reshape(rows, k // 32, 32)).max(axis=2)
    assert np.array_equal(s, amax / np.float32(127))
    assert (np.abs(hi.reshape(rows, k // 32, 32)).max(axis=2) == 127).all()
    # sign symmetry and power-of-two scaling
    hn, ln, sn = oracle.quantize_act("i8x2", -x)
    assert np.array_equal(hn, -hi) and np.array_equal(ln, -lo) and np.array_equal(sn, s)
    for p in (-7, 5):
        hp, lp, sp = oracle.quantize_act("i8x2", np.ldexp(x, p))
        assert np.array_equal(hp, hi) and np.array_equal(lp, lo)
        assert np.array_equal(sp, np.ldexp(s, p))


# ------------------------------------------------- brute force and error bounds

@pytest.mark.parametrize("n,k,rows,seed", [(5, 64, 1, 11), (17, 128, 3, 12), (64, 256, 2, 13),
                                           (33, 96, 4, 14)])
def test_projection_against_brute_force(n, k, rows, seed):
    w = synth.weights(n, k, seed=seed, outlier_frac=0.1)
    x = synth.activations(rows, k, seed=seed + 50, outlier_frac=0.05)
    res = synth.normal(seed + 60, (rows, n))
    blocks = oracle.quantize_weights(w)
    wd = oracle.dequantize_weights(blocks, n, k)
    # dequantized weights against numpy's own decode of the bytes
    scales, q = oracle.split_blocks(blocks, n, k)
    dq = np.repeat(scales.view(np.float16).astype(np.float64), 32, axis=1)
    assert np.array_equal(wd, dq * q)
    x64 = x.astype(np.float64)
    for mode in ("f32", "i8", "i8x2"):
        if mode == "f32":
            y, a = oracle.project(mode, blocks, n, k, rows, x=x, residual=res)
            v = x64
        else:
            hi, lo, s = oracle.quantize_act(mode, x)
            y, a = oracle.project(mode, blocks, n, k, rows, hi=hi, lo=lo, scale=s, residual=res)
            se = np.repeat(s.astype(np.float64), 32, axis=1)
            v = se * hi if mode == "i8" else se * (hi + lo / 128.0)
        brute = oracle.dense_matvec(wd, v) + res.astype(np.float64)
        np_ref = v @ wd.T + res.astype(np.float64)
        assert (np.abs(y - brute) <= 1e-12 * a).all(), mode
        assert (np.abs(y - np_ref) <= 1e-12 * a).all(), mode
        if mode != "f32":
            # closed-form bound of the activation rounding against unquantized x:
            # |sum_b d s (q . e_b)| <= sum_b d s (1/2 or 1/256) sum_j |q_j|
            exact_x = oracle.dense_matvec(wd, x64) + res.astype(np.float64)
            step = 0.5 if mode == "i8" else 1.0 / 256
            qa = np.abs(q).reshape(n, k // 32, 32).sum(axis=2).astype(np.float64)
            ds = scales.view(np.float16).astype(np.float64)
            bound = np.einsum("nb,rb->rn", ds * qa, s.astype(np.float64)) * (step + 2.0 ** -15)
            assert (np.abs(y - exact_x) <= bound + 1e-12 * a).all(), mode
    # the quantized projection approximates the unquantized f64 product within the
    # weight-rounding plus activation-rounding bound
    y_true = oracle.dense_matvec(w.astype(np.float64), x64) + res.astype(np.float64)
    hi, lo, s = oracle.quantize_act("i8x2", x)
    y2, a2 = oracle.project("i8x2", blocks, n, k, rows, hi=hi, lo=lo, scale=s, residual=res)
    v2 = np.repeat(s.astype(np.float64), 32, axis=1) * (hi + lo / 128.0)
    bound = np.abs(x64) @ np.abs(w.astype(np.float64) - wd).T + np.abs(x64 - v2) @ np.abs(wd).T
    assert (np.abs(y2 - y_true) <= bound * (1 + 1e-9) + 1e-12 * a2).all()


def test_project_at_matches_project():
    n, k, rows = 50, 512, 3
    w = synth.weights(n, k, seed=21)
    x = synth.activations(rows, k, seed=22)
    blocks = oracle.quantize_weights(w)
    hi, lo, s = oracle.quantize_act("i8x2", x)
    y, a = oracle.project("i8x2", blocks, n, k, rows, hi=hi, lo=lo, scale=s)
    ri = np.array([0, 2, 1, 2], np.int64)
    ni = np.array([0, 49, 17, 3], np.int64)
    ys, as_ = oracle.project_at("i8x2", blocks, n, k, rows, ri, ni, hi=hi, lo=lo, scale=s)
    assert np.array_equal(ys, y[ri, ni]) and np.array_equal(as_, a[ri, ni])


def test_modes_agree_to_their_precision():
    """The three numerics estimate one product: the two-word result is within
    ~2^-8 of the activation step of the f32-mode result, the one-word within 1/2."""
    call = workloads.tiny()[0]
    w = call.make_weights()[:32]
    x = call.make_activations()
    blocks = oracle.quantize_weights(w)
    y0, a0 = oracle.project("f32", blocks, 32, call.k, 1, x=x)
    for mode, step in (("i8", 0.5), ("i8x2", 1.0 / 256)):
        hi, lo, s = oracle.quantize_act(mode, x)
        y, _ = oracle.project(mode, blocks, 32, call.k, 1, hi=hi, lo=lo, scale=s)
        scales, q = oracle.split_blocks(blocks, 32, call.k)
        qa = np.abs(q).reshape(32, -1, 32).sum(axis=2)
        bound = (scales.view(np.float16).astype(np.float64) * qa) @ s[0].astype(np.float64) * (step + 2.0 ** -15)
        assert (np.abs(y[0] - y0[0]) <= bound + 1e-12 * a0[0]).all()


def _error_scale_numpy(mode, blocks, n, k, x, residual):
    """A = sum_b |block term| + |residual|, written independently of the oracle:
    the block sums from numpy's int64 einsum (integer modes) or f64 einsum (f32
    mode), every block term formed in f64 from the block's binary16 and f32
    scales as numpy decodes them."""
    scales, q = oracle.split_blocks(blocks, n, k)
    d = scales.view(np.float16).astype(np.float64)                    # [n][nb]
    qb = q.reshape(n, k // 32, 32)
    if mode == "f32":
        xb = x.astype(np.float64).reshape(x.shape[0], k // 32, 32)
        terms = d[None] * np.einsum("nbj,rbj->rnb", qb.astype(np.float64), xb)
    else:
        hi, lo, s = oracle.quantize_act(mode, x)
        rows = x.shape[0]
        sh = np.einsum("nbj,rbj->rnb", qb.astype(np.int64), hi.reshape(rows, k // 32, 32).astype(np.int64))
        t = sh.astype(np.float64)
        if mode == "i8x2":
            sl = np.einsum("nbj,rbj->rnb", qb.astype(np.int64), lo.reshape(rows, k // 32, 32).astype(np.int64))
            t = t + sl.astype(np.float64) / 128.0
        terms = d[None] * s.astype(np.float64)[:, None, :] * t
    a = np.abs(terms).sum(axis=2)
    if residual is not None:
        a = a + np.abs(residual.astype(np.float64))
    return a


@pytest.mark.parametrize("mode", ["f32", "i8", "i8x2"])
@pytest.mark.parametrize("n,k,rows,seed,with_res", [(17, 128, 3, 31, True), (40, 1024, 2, 32, False),
                                                    (9, 4096, 1, 33, True)])
def test_error_scale_pinned_from_both_sides(mode, n, k, rows, seed, with_res):
    """The oracle's error scale A (which sets the floor of every parity gate)
    equals an independent numpy computation of sum_b |block term| + |residual|
    up to summation order (relative 1e-12), so it can be neither inflated nor
    shrunk without failing here."""
    w = synth.weights(n, k, seed=seed, outlier_frac=0.1)
    x = synth.activations(rows, k, seed=seed + 1, outlier_frac=0.05)
    res = synth.normal(seed + 2, (rows, n)) if with_res else None
    blocks = oracle.quantize_weights(w)
    if mode == "f32":
        _, a = oracle.project(mode, blocks, n, k, rows, x=x, residual=res)
    else:
        hi, lo, s = oracle.quantize_act(mode, x)
        _, a = oracle.project(mode, blocks, n, k, rows, hi=hi, lo=lo, scale=s, residual=res)
    ref = _error_scale_numpy(mode, blocks, n, k, x, res)
    assert np.allclose(a, ref, rtol=1e-12, atol=0.0), float(np.max(np.abs(a / ref - 1)))
