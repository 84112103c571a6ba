"""Seeded random sweep over every projection entry point, against the CPU oracle.

Each case draws an entry point (q8_matmul_rows, q8_matmul_rows_ws, and at one
row q8_matvec and q8_matvec_argmax; q8_block_sums in the integer modes), an
activation mode, a shape (1..130 rows, k any multiple of 64, n from 1 to
20000), a residual (none, separate, or in place in y) and, for integer stacks
of at most 8 rows, whether the stack is passed as f32 x and quantized inside
the call.  Outputs pass helpers.gate against the oracle; block sums match bit
for bit; the arg-max is the lowest index of the largest output; the K-split
counters are back at zero after each call that shares the one workspace.
"""
import math
import random

import numpy as np
import pytest
import torch

import oracle
import q8_projection_amd as q8
import synth

from helpers import gate, say

pytestmark = pytest.mark.gpu

CASES = 300
SEED = 2024


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(rng):
    mode = rng.choice(["f32", "i8", "i8x2"])
    u = rng.random()
    if u < 0.3:
        rows = 1
    elif u < 0.6:
        rows = rng.randint(2, 8)
    elif u < 0.85:
        rows = rng.randint(9, 64)
    else:
        rows = rng.randint(65, 130)
    k = 64 * rng.randint(1, 256)
    if rng.random() < 0.5:
        k = 256 * max(1, k // 256)
    if rng.random() < 0.5:
        n = max(1, int(math.exp(rng.uniform(0, math.log(20000)))))
    else:
        n = rng.randint(1000, 20000)
    while n * k * rows > 4096 * 14336 * 24:
        n = max(1, n // 2)
    entries = ["matmul_rows", "matmul_rows_ws"]
    if rows == 1:
        entries += ["matvec", "matvec_argmax"]
    if mode != "f32":
        entries.append("block_sums")
    entry = rng.choice(entries)
    if entry == "block_sums":
        while rows * n * (k // 32) * 2 > (48 << 20):
            n = max(1, n // 2)
    residual = "none" if entry == "block_sums" else rng.choice(["none", "separate", "inplace"])
    inside = (mode != "f32" and rows <= 8 and entry in ("matmul_rows", "matmul_rows_ws", "matvec")
              and rng.random() < 0.25)
    return entry, mode, n, k, rows, residual, inside


def test_random_entry_points():
    torch.cuda.set_device(0)
    q8.lib()
    rng = random.Random(SEED)
    workspace = torch.zeros(96 << 20, dtype=torch.uint8, device="cuda")
    counters = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    for i in range(CASES):
        entry, mode, n, k, rows, residual, inside = _case(rng)
        say("sweep", i, entry, mode, n, k, rows, residual, "inside" if inside else "")
        w = synth.weights(n, k, seed=10000 + i, outlier_frac=0.05)
        x = synth.activations(rows, k, seed=20000 + i, outlier_frac=0.05)
        blocks = oracle.quantize_weights(w)
        wd = _dev(blocks)
        res = synth.normal(30000 + i, (rows, n)) if residual != "none" else None
        hi = lo = sc = None
        if mode != "f32":
            hi, lo, sc = oracle.quantize_act(mode, x)
        what = f"case {i} {entry} {mode} {n}x{k} rows={rows} residual={residual}"
        if entry == "block_sums":
            got = q8.block_sums(mode, wd, n, k, _dev(hi), None if lo is None else _dev(lo), rows=rows)
            torch.cuda.synchronize()
            assert np.array_equal(got.cpu().numpy(), oracle.block_sums(mode, blocks, n, k, hi, lo)), what
            continue
        kw = {}
        if mode == "f32" or inside:
            kw["x"] = _dev(x)
        else:
            kw.update(hi=_dev(hi), lo=None if lo is None else _dev(lo), scale=_dev(sc))
        out = None
        if residual == "separate":
            kw["residual"] = _dev(res)
        elif residual == "inplace":
            out = _dev(res)
            kw["residual"] = out
        if entry in ("matvec", "matvec_argmax"):
            kw = {key: (v.view(-1) if v is not None else None) for key, v in kw.items()}
            out = None if out is None else kw["residual"]
        idx = None
        if entry == "matmul_rows":
            y = q8.matmul_rows(mode, wd, n, k, out=out, rows=rows, **kw)
        elif entry == "matmul_rows_ws":
            need = q8.matmul_rows_workspace_bytes(mode, n, k, rows)
            assert need <= workspace.numel(), what
            y = q8.matmul_rows_ws(mode, wd, n, k, out=out, rows=rows, workspace=workspace if need else None, **kw)
        elif entry == "matvec":
            y = q8.matvec(mode, wd, n, k, out=out, **kw)
        else:
            y, idx = q8.matvec_argmax(mode, wd, n, k, out=out, **kw)
        torch.cuda.synchronize()
        yh = y.cpu().numpy().reshape(rows, n)
        if mode == "f32":
            r, a = oracle.project(mode, blocks, n, k, rows, x=x, residual=res)
        else:
            r, a = oracle.project(mode, blocks, n, k, rows, hi=hi, lo=lo, scale=sc, residual=res)
        gate(yh, r, a, what)
        if idx is not None:
            v = yh.ravel()
            assert int(idx.cpu().item()) == int(np.flatnonzero(v == v.max())[0]), what
        if entry == "matmul_rows_ws":
            assert int(workspace[:counters].count_nonzero().item()) == 0, what
