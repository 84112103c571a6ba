"""Graph capture and replay of a decode step's projections (codegen_cuda::lane
page, description: a step is recorded as a graph one time and that graph re-run for every token).

The library enqueues only kernels (no allocation, copy, memset or host
synchronization), so a sequence of calls captured into a HIP graph must
reproduce its results on every replay, with unrelated eager work and
synchronizations in between.  Every replay is checked against the CPU oracle
(quantized activations bit for bit, outputs within the gate), not only against
the eager run."""
import numpy as np
import pytest
import torch

import oracle
import q8_projection_amd as q8
import synth
from helpers import gate, say
from synth import workloads

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _expected(mode, blocks, n, k, x, res):
    hi, lo, sc = oracle.quantize_act(mode, x)
    r, a = oracle.project(mode, blocks, n, k, x.shape[0], hi=hi, lo=lo, scale=sc, residual=res)
    return (hi, lo, sc), r, a


def test_step_graph_replays_match_eager_and_oracle():
    torch.cuda.set_device(0)
    say("graph replay: rows 1 / 2 / 8 / 64, both integer modes, residual")
    shapes = [  # (n, k, rows, mode, residual)
        (1024, 2048, 1, "i8x2", True),   # GEMV, LDS ring
        (777, 1024, 2, "i8", False),     # GEMV, two rows
        (2048, 4096, 8, "i8x2", True),   # MFMA, one activation tile
        (1500, 1024, 64, "i8", False),   # MFMA, four activation tiles
    ]
    bufs, want = [], []
    for i, (n, k, rows, mode, with_res) in enumerate(shapes):
        blocks = oracle.quantize_weights(synth.weights(n, k, seed=1100 + i))
        xh = synth.activations(rows, k, seed=1200 + i)
        resh = synth.normal(1300 + i, (rows, n)) if with_res else None
        want.append(_expected(mode, blocks, n, k, xh, resh))
        w, x = _dev(blocks), _dev(xh)
        res = None if resh is None else _dev(resh)
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
    g = _capture(step)

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
        for (n, k, rows, mode, *_), r, b, (q, rr, aa) in zip(shapes, ref, bufs, want):
            assert torch.equal(b[-1], r), (replay, n, k, rows, mode)
            assert np.array_equal(b[7].cpu().numpy(), q[0]), (replay, n, "hi")
            if mode == "i8x2":
                assert np.array_equal(b[8].cpu().numpy(), q[1]), (replay, n, "lo")
            gate(b[-1].cpu().numpy(), rr, aa, f"replay {replay} {n}x{k} rows={rows} {mode}")
    assert float(scratch[0]) == 4.0


def test_decode_layer_graph_against_the_oracle():
    """One decode layer's projections at one row, two-word (model::author page,
    Functions: decode_layer): fused QKV 6144x4096, O 4096x4096 with the
    residual, gate and up 14336x4096 on one shared input, down 4096x14336 with
    the residual -- four activation quantizations and five projections captured
    once into a HIP graph and replayed.  Every replay's quantized inputs equal
    the oracle's bit for bit and every output meets the oracle's gate."""
    torch.cuda.set_device(0)
    calls = workloads.decode_layer()
    say("decode layer graph:", ", ".join(f"{c.name} {c.n}x{c.k}" for c in calls))
    inputs, want_q = {}, {}
    for c in calls:
        if c.x_seed not in inputs:
            xh = c.make_activations()
            want_q[c.x_seed] = oracle.quantize_act("i8x2", xh)
            inputs[c.x_seed] = (_dev(xh), torch.empty((1, c.k), dtype=torch.int8, device="cuda"),
                                torch.empty((1, c.k), dtype=torch.int8, device="cuda"),
                                torch.empty((1, c.k // 32), dtype=torch.float32, device="cuda"))
    bufs, want = [], []
    for c in calls:
        blocks = oracle.quantize_weights(c.make_weights())
        resh = c.make_residual()
        hi, lo, sc = want_q[c.x_seed]
        r, a = oracle.project("i8x2", blocks, c.n, c.k, 1, hi=hi, lo=lo, scale=sc, residual=resh)
        want.append((r, a))
        bufs.append((c, _dev(blocks), None if resh is None else _dev(resh),
                     torch.empty((1, c.n), dtype=torch.float32, device="cuda")))

    def layer():
        done = set()
        for c, w, res, y in bufs:
            x, hi, lo, sc = inputs[c.x_seed]
            if c.x_seed not in done:  # gate and up share one quantized input
                q8.quantize_act("i8x2", x, hi=hi, lo=lo, scale=sc)
                done.add(c.x_seed)
            q8.matvec("i8x2", w, c.n, c.k, hi=hi[0], lo=lo[0], scale=sc[0],
                      residual=None if res is None else res[0], out=y[0])

    g = _capture(layer)
    scratch = torch.zeros(1 << 20, device="cuda")
    for replay in range(3):
        for _, _, _, y in bufs:
            y.fill_(float("nan"))
        for _, hi, lo, sc in inputs.values():
            hi.zero_()
            lo.zero_()
            sc.zero_()
        scratch.add_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for seed, (_, hi, lo, sc) in inputs.items():
            qh, ql, qs = want_q[seed]
            assert np.array_equal(hi.cpu().numpy(), qh) and np.array_equal(lo.cpu().numpy(), ql), (replay, seed)
            assert np.array_equal(sc.cpu().numpy().view(np.uint32), qs.view(np.uint32)), (replay, seed)
        for (c, _, _, y), (r, a) in zip(bufs, want):
            rel, ulps = gate(y.cpu().numpy(), r, a, f"decode layer replay {replay} {c.name}")
            say("decode layer", replay, c.name, f"max rel err {rel:.3g}", f"max ulps {ulps}")
    assert float(scratch[0]) == 3.0
