"""Graph capture and replay of a decode step's projections (codegen_cuda::lane
page, description: each step is captured once as a graph and replayed per token).

The library enqueues only kernels (no allocation, copy, memset or host
synchronization), so a sequence of calls captured into a HIP graph must
reproduce the eager results bit for bit on every replay, with unrelated eager
work and synchronizations in between."""
import numpy as np
import pytest
import torch

import oracle
import q8_projection_amd as q8
import synth
from helpers import say

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_step_graph_replays_match_eager():
    torch.cuda.set_device(0)
    say("graph replay: rows 1 / 2 / 8 / 64, both integer modes, residual")
    shapes = [  # (n, k, rows, mode, residual)
        (1024, 2048, 1, "i8x2", True),   # GEMV, LDS ring
        (777, 1024, 2, "i8", False),     # GEMV, two rows
        (2048, 4096, 8, "i8x2", True),   # MFMA, one activation tile
        (1500, 1024, 64, "i8", False),   # MFMA, four activation tiles
    ]
    bufs = []
    for i, (n, k, rows, mode, with_res) in enumerate(shapes):
        w = _dev(oracle.quantize_weights(synth.weights(n, k, seed=1100 + i)))
        x = _dev(synth.activations(rows, k, seed=1200 + i))
        res = _dev(synth.normal(1300 + i, (rows, n))) if with_res else None
        hi = torch.empty((rows, k), dtype=torch.int8, device="cuda")
        lo = torch.empty((rows, k), dtype=torch.int8, device="cuda") if mode == "i8x2" else None
        sc = torch.empty((rows, k // 32), dtype=torch.float32, device="cuda")
        y = torch.empty((rows, n), dtype=torch.float32, device="cuda")
        bufs.append((n, k, rows, mode, w, x, res, hi, lo, sc, y))

    def step():
        for n, k, rows, mode, w, x, res, hi, lo, sc, y in bufs:
            q8.quantize_act(mode, x, hi=hi, lo=lo, scale=sc)
            q8.matmul_rows(mode, w, n, k, hi=hi, lo=lo, scale=sc, residual=res, out=y)

    step()
    torch.cuda.synchronize()
    ref = [b[-1].clone() for b in bufs]

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    scratch = torch.zeros(1 << 20, device="cuda")
    for replay in range(4):
        for b in bufs:
            b[-1].fill_(float("nan"))
            for t in (b[7], b[8], b[9]):
                if t is not None:
                    t.zero_()
        scratch.add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (n, k, rows, mode, *_), r, b in zip(shapes, ref, bufs):
            assert torch.equal(b[-1], r), (replay, n, k, rows, mode)
    assert float(scratch[0]) == 4.0
