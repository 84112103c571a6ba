"""The K-split projection (q8_matmul_rows_ws) against the CPU oracle, on the GPU.

A short integer stack on a matrix of at most 16 rows per CU (a batched decode
step's down projection, model::author page, Functions: decode_batch) is split
over workgroups along K; the partial sums of a 64-row range meet in a caller
workspace and the last workgroup to arrive adds them in split order.  Checked
here: the gate against the oracle at full size and on ragged and tiny shapes,
bitwise equal results from call to call (the order of arrival does not show),
counters left at zero, in-place residual, one workspace shared by calls of
different shapes, graph replays, and the calls that do not split (which are
q8_matmul_rows's, bit for bit)."""
import numpy as np
import pytest
import torch

import oracle
import q8_projection_amd as q8
import synth
from helpers import gate, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    torch.cuda.set_device(0)
    q8.lib()
    yield


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(n, k, rows, mode, with_res, seed):
    blocks = oracle.quantize_weights(synth.weights(n, k, seed=seed))
    x = synth.activations(rows, k, seed=seed + 1)
    res = synth.normal(seed + 2, (rows, n)) if with_res else None
    return blocks, x, res


def _expected(mode, blocks, n, k, x, res):
    if mode == "f32":
        return oracle.project(mode, blocks, n, k, x.shape[0], x=x, residual=res)
    hi, lo, sc = oracle.quantize_act(mode, x)
    return oracle.project(mode, blocks, n, k, x.shape[0], hi=hi, lo=lo, scale=sc, residual=res)


def _stack(mode, xd):
    """The stack's arguments to a projection: x itself in the f32 mode, else
    its quantization on the GPU."""
    if mode == "f32":
        return {"x": xd}
    hi, lo, sc = q8.quantize_act(mode, xd)
    return {"hi": hi, "lo": lo, "scale": sc}


def _counters_zero(ws, n):
    """The counters of every range a splitting matrix can have (16 rows per CU)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    count_bytes = ((16 * cus + 63) // 64 * 4 + 15) // 16 * 16
    return int(ws[:count_bytes].view(torch.int32).abs().sum()) == 0


# (n, k, rows, mode, residual).  One activation tile, stacks of at least 400 KB
# (rows x k, twice in two-word mode) or at most 8 rows per CU: 4096 x 28672 at
# 8 two-word rows and 16 one-word rows; 8 one-word rows in the two-word layout;
# the smallest k that splits; 1000 rows (K in 8 parts); a ragged last range
# (4090 = 63 x 64 + 58); 2048 rows; two rows on a long K; 130, 33 and 1 rows;
# 2048 x 14336 at 2 two-word and 5 one-word rows.  Several tiles: the down
# projection 4096 x 14336 at 16 two-word rows (two tiles), 33 and 64 one-word
# rows (four), 64 two-word rows (eight); 50 two-word rows of 2000 x 14336
# (eight tiles, the last half empty); 25 one-word rows on a ragged n.  More
# than 64 rows: 100 two-word rows (two split slices), 70 one-word rows (a
# split slice, then 6 rows that do not split).  The f32 mode (f64 matrix
# cores, two weight tiles a workgroup): 16 rows of 4096 x 8192, 64 of 4096 x
# 4096, 24 rows of 2048 x 14336, 5 rows on a ragged n, 33 rows, and 100 rows
# in two slices.
_CASES = [(4096, 28672, 8, "i8x2", True), (4096, 28672, 16, "i8", False), (4096, 57344, 8, "i8", True),
          (4096, 25600, 8, "i8x2", False), (1000, 28672, 8, "i8x2", True), (4090, 28672, 8, "i8x2", True),
          (4090, 28672, 15, "i8", False), (2048, 32768, 7, "i8x2", True), (512, 131072, 2, "i8x2", True),
          (130, 57344, 8, "i8x2", True), (33, 65536, 4, "i8x2", True), (1, 32768, 8, "i8x2", False),
          (2048, 14336, 2, "i8x2", True), (2048, 14336, 5, "i8", False),
          (4096, 14336, 16, "i8x2", True), (4096, 14336, 33, "i8", True), (4096, 14336, 64, "i8", False),
          (4096, 14336, 64, "i8x2", True), (2000, 14336, 50, "i8x2", False), (4090, 16384, 25, "i8", True),
          (4096, 14336, 100, "i8x2", True), (4096, 14336, 70, "i8", False),
          (4096, 8192, 16, "f32", True), (4096, 4096, 64, "f32", False), (2048, 14336, 24, "f32", True),
          (4090, 8192, 5, "f32", True), (1000, 8192, 33, "f32", False), (4096, 14336, 100, "f32", True)]


@pytest.mark.parametrize("n,k,rows,mode,with_res", _CASES)
def test_split_parity(n, k, rows, mode, with_res):
    need = q8.matmul_rows_workspace_bytes(mode, n, k, rows)
    say("k split", n, k, rows, mode, with_res, "workspace", need)
    assert need > 0, "this shape splits K"
    blocks, x, res = _case(n, k, rows, mode, with_res, seed=1500 + n % 101 + rows)
    w = _dev(blocks)
    act = _stack(mode, _dev(x))
    resd = None if res is None else _dev(res)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    y = q8.matmul_rows_ws(mode, w, n, k, residual=resd, workspace=ws, **act)
    torch.cuda.synchronize()
    assert _counters_zero(ws, n)
    r, a = _expected(mode, blocks, n, k, x, res)
    gate(y.cpu().numpy(), r, a, f"k split {n}x{k} rows={rows} {mode}")
    # the same bits on every call, whatever order the workgroups arrive in
    for _ in range(3):
        y2 = q8.matmul_rows_ws(mode, w, n, k, residual=resd, workspace=ws, **act)
        torch.cuda.synchronize()
        assert torch.equal(y2, y)
    assert _counters_zero(ws, n)
    # the unsplit projection passes the same gate; the two differ at most in
    # the last bits of some outputs (f64 partials added in another order)
    yu = q8.matmul_rows(mode, w, n, k, residual=resd, **act)
    torch.cuda.synchronize()
    gate(yu.cpu().numpy(), r, a, f"unsplit {n}x{k} rows={rows} {mode}")


def test_split_inplace_residual():
    n, k, rows, mode = 4096, 28672, 8, "i8x2"
    say("k split in place", n, k, rows, mode)
    blocks, x, res = _case(n, k, rows, mode, True, seed=1700)
    w = _dev(blocks)
    hi, lo, sc = q8.quantize_act(mode, _dev(x))
    ws = torch.zeros(q8.matmul_rows_workspace_bytes(mode, n, k, rows), dtype=torch.uint8, device="cuda")
    ref = q8.matmul_rows_ws(mode, w, n, k, hi=hi, lo=lo, scale=sc, residual=_dev(res), workspace=ws)
    h = _dev(res)
    q8.matmul_rows_ws(mode, w, n, k, hi=hi, lo=lo, scale=sc, residual=h, out=h, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(h, ref)
    r, a = _expected(mode, blocks, n, k, x, res)
    gate(h.cpu().numpy(), r, a, "k split in place")


def test_one_workspace_for_calls_of_different_shapes():
    """Calls in a row on one workspace, with fewer, then more, then fewer row
    ranges (the partials of one call cover bytes that are counters of no
    other); every call equals its own run on a fresh zero-filled workspace."""
    shapes = [(300, 28672, 8, "i8x2"), (4096, 14336, 64, "i8x2"), (2000, 32768, 7, "i8x2"),
              (4096, 14336, 33, "i8"), (33, 28672, 16, "i8")]
    big = max(q8.matmul_rows_workspace_bytes(m, n, k, r) for n, k, r, m in shapes)
    shared = torch.zeros(big, dtype=torch.uint8, device="cuda")
    for i, (n, k, rows, mode) in enumerate(shapes):
        say("shared workspace", n, k, rows, mode)
        blocks, x, _ = _case(n, k, rows, mode, False, seed=1800 + i)
        w = _dev(blocks)
        hi, lo, sc = q8.quantize_act(mode, _dev(x))
        y = q8.matmul_rows_ws(mode, w, n, k, hi=hi, lo=lo, scale=sc, workspace=shared)
        fresh = torch.zeros(q8.matmul_rows_workspace_bytes(mode, n, k, rows), dtype=torch.uint8, device="cuda")
        yf = q8.matmul_rows_ws(mode, w, n, k, hi=hi, lo=lo, scale=sc, workspace=fresh)
        torch.cuda.synchronize()
        assert torch.equal(y, yf)
        assert _counters_zero(shared, n)
        r, a = _expected(mode, blocks, n, k, x, None)
        gate(y.cpu().numpy(), r, a, f"shared workspace {n}x{k} rows={rows} {mode}")


@pytest.mark.parametrize("n,k,rows,mode", [(14336, 2048, 8, "i8x2"), (4096, 28672, 1, "i8x2"),
                                           (4096, 14336, 16, "i8"), (4096, 4096, 48, "i8x2"),
                                           (4096, 28672 - 64, 8, "i8x2"), (4096, 14336, 8, "i8x2"),
                                           (4096, 28672, 8, "i8")])
def test_calls_that_do_not_split_are_matmul_rows(n, k, rows, mode):
    """No workspace needed: the call is q8_matmul_rows's, bit for bit, and a
    workspace passed anyway is neither read nor written."""
    say("no split", n, k, rows, mode)
    assert q8.matmul_rows_workspace_bytes(mode, n, k, rows) == 0
    blocks, x, _ = _case(n, k, rows, mode, False, seed=1900 + rows)
    w = _dev(blocks)
    hi, lo, sc = q8.quantize_act(mode, _dev(x))
    ws = torch.full((4096,), 7, dtype=torch.uint8, device="cuda")
    y = q8.matmul_rows_ws(mode, w, n, k, hi=hi, lo=lo, scale=sc, workspace=ws)
    yu = q8.matmul_rows(mode, w, n, k, hi=hi, lo=lo, scale=sc)
    torch.cuda.synchronize()
    assert torch.equal(y, yu)
    assert bool((ws == 7).all())


def test_split_inside_quantization_is_matmul_rows():
    """A stack given as x is quantized inside the GEMV: no split, the workspace
    untouched, the result that of q8_matmul_rows."""
    n, k, rows, mode = 4096, 28672, 8, "i8x2"
    say("k split with x", n, k, rows, mode)
    blocks, x, _ = _case(n, k, rows, mode, False, seed=1950)
    w, xd = _dev(blocks), _dev(x)
    ws = torch.zeros(q8.matmul_rows_workspace_bytes(mode, n, k, rows), dtype=torch.uint8, device="cuda")
    ws[:16] = 5
    y = q8.matmul_rows_ws(mode, w, n, k, x=xd, workspace=ws)
    yu = q8.matmul_rows(mode, w, n, k, x=xd)
    torch.cuda.synchronize()
    assert torch.equal(y, yu)
    assert int(ws[:16].sum()) == 16 * 5 and int(ws[16:].sum()) == 0


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


def test_split_graph_replays():
    """Quantization and four split projections (one in the f32 mode) captured
    once and replayed four times with eager work between replays: every replay
    equals the eager run bit for bit and passes the gate; counters stay zero."""
    shapes = [(4096, 28672, 8, "i8x2", True), (1000, 28672, 16, "i8", False), (4096, 14336, 64, "i8x2", True),
              (4096, 4096, 24, "f32", True)]
    bufs, want = [], []
    for i, (n, k, rows, mode, with_res) in enumerate(shapes):
        blocks, x, res = _case(n, k, rows, mode, with_res, seed=2000 + i)
        want.append(_expected(mode, blocks, n, k, x, res))
        hi = torch.empty((rows, k), dtype=torch.int8, device="cuda")
        lo = torch.empty((rows, k), dtype=torch.int8, device="cuda") if mode == "i8x2" else None
        sc = torch.empty((rows, k // 32), dtype=torch.float32, device="cuda")
        ws = torch.zeros(q8.matmul_rows_workspace_bytes(mode, n, k, rows), dtype=torch.uint8, device="cuda")
        y = torch.empty((rows, n), dtype=torch.float32, device="cuda")
        bufs.append((n, k, rows, mode, _dev(blocks), _dev(x), None if res is None else _dev(res), hi, lo, sc, ws, y))

    def step():
        for n, k, rows, mode, w, x, res, hi, lo, sc, ws, y in bufs:
            if mode == "f32":
                q8.matmul_rows_ws(mode, w, n, k, x=x, residual=res, out=y, workspace=ws)
                continue
            q8.quantize_act(mode, x, hi=hi, lo=lo, scale=sc)
            q8.matmul_rows_ws(mode, w, n, k, hi=hi, lo=lo, scale=sc, residual=res, out=y, workspace=ws)

    say("k split graph: capture")
    step()
    torch.cuda.synchronize()
    ref = [b[-1].clone() for b in bufs]
    g = _capture(step)
    other = torch.zeros(1 << 20, device="cuda")
    for replay in range(4):
        for b in bufs:
            b[-1].fill_(float("nan"))
        other.add_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("k split graph: replay", replay)
        for (n, k, rows, mode, _), r, b, (rr, aa) in zip(shapes, ref, bufs, want):
            assert torch.equal(b[-1], r), (replay, n, k, rows, mode)
            assert _counters_zero(b[10], n)
            gate(b[-1].cpu().numpy(), rr, aa, f"split replay {replay} {n}x{k} rows={rows} {mode}")
    assert float(other[0]) == 4.0


def test_split_misaligned_weights_run_unsplit():
    """Weights that q8_matmul_rows cannot give its matrix-core kernels (4-byte
    but not 16-byte aligned) run on q8_matmul_rows's path, bit for bit, and
    leave the workspace alone."""
    n, k, rows, mode = 4096, 14336, 16, "i8x2"
    say("k split, misaligned weights", n, k, rows, mode)
    blocks, x, _ = _case(n, k, rows, mode, False, seed=2100)
    nbytes = blocks.size
    wbuf = torch.empty(nbytes + 16, dtype=torch.uint8, device="cuda")
    wbuf[4:4 + nbytes].copy_(_dev(blocks).reshape(-1))
    w4 = wbuf[4:4 + nbytes]
    hi, lo, sc = q8.quantize_act(mode, _dev(x))
    need = q8.matmul_rows_workspace_bytes(mode, n, k, rows)
    assert need > 0
    ws = torch.full((need,), 3, dtype=torch.uint8, device="cuda")
    y = q8.matmul_rows_ws(mode, w4, n, k, hi=hi, lo=lo, scale=sc, workspace=ws)
    yu = q8.matmul_rows(mode, w4, n, k, hi=hi, lo=lo, scale=sc)
    torch.cuda.synchronize()
    assert torch.equal(y, yu)
    assert bool((ws == 3).all())
    r, a = _expected(mode, blocks, n, k, x, None)
    gate(y.cpu().numpy(), r, a, "k split, misaligned weights")


def test_split_calls_queued_back_to_back():
    """48 split calls of varying shapes and modes queued on one stream, sharing
    one workspace, with no host synchronization between them: every output
    equals the same call run alone (the counters each call leaves at zero are
    what the next one starts from)."""
    shapes = [(4096, 14336, 16, "i8x2"), (2048, 14336, 5, "i8"), (1000, 8192, 33, "f32"),
              (4096, 14336, 64, "i8"), (512, 131072, 2, "i8x2"), (4096, 8192, 24, "f32")]
    cases = []
    for i, (n, k, rows, mode) in enumerate(shapes):
        assert q8.matmul_rows_workspace_bytes(mode, n, k, rows) > 0, (n, k, rows, mode)
        blocks, x, _ = _case(n, k, rows, mode, False, seed=2200 + i)
        cases.append((n, k, rows, mode, _dev(blocks), _stack(mode, _dev(x))))
    big = max(q8.matmul_rows_workspace_bytes(m, n, k, r) for n, k, r, m in shapes)
    shared = torch.zeros(big, dtype=torch.uint8, device="cuda")
    say("k split, 48 calls queued")
    order = [i % len(cases) for i in range(48)]
    outs = []
    for i in order:
        n, k, rows, mode, w, act = cases[i]
        outs.append(q8.matmul_rows_ws(mode, w, n, k, workspace=shared, **act))
    torch.cuda.synchronize()
    assert _counters_zero(shared, 0)
    for i, (n, k, rows, mode, w, act) in enumerate(cases):
        fresh = torch.zeros(q8.matmul_rows_workspace_bytes(mode, n, k, rows), dtype=torch.uint8, device="cuda")
        ref = q8.matmul_rows_ws(mode, w, n, k, workspace=fresh, **act)
        torch.cuda.synchronize()
        for j, o in zip(order, outs):
            if j == i:
                assert torch.equal(o, ref), (n, k, rows, mode)


def _random_split_shapes(count, seed):
    """Seeded (n, k, rows, mode, residual) draws, kept to those the library
    splits, every stack under 4096 x 14336 x 24 multiply-adds."""
    import random
    rng = random.Random(seed)
    out = []
    while len(out) < count:
        mode = rng.choice(["i8", "i8x2", "f32"])
        n = rng.choice([rng.randint(1, 4096), rng.randint(1, 1024), rng.randint(3000, 4096)])
        k = 256 * rng.randint(4, 112) if mode != "f32" else 64 * rng.randint(8, 400)
        rows = rng.randint(2, 70)
        if n * k * rows > 4096 * 14336 * 24 or q8.matmul_rows_workspace_bytes(mode, n, k, rows) == 0:
            continue
        out.append((n, k, rows, mode, rng.random() < 0.5))
    return out


def test_split_random_shapes():
    """Sixteen seeded random shapes that split (all three modes, ragged n and
    k, 2..70 rows): the gate against the oracle, the same bits twice, counters
    back at zero."""
    for i, (n, k, rows, mode, with_res) in enumerate(_random_split_shapes(16, seed=12345)):
        say("k split random", i, n, k, rows, mode, with_res)
        blocks, x, res = _case(n, k, rows, mode, with_res, seed=3000 + i)
        w = _dev(blocks)
        act = _stack(mode, _dev(x))
        resd = None if res is None else _dev(res)
        ws = torch.zeros(q8.matmul_rows_workspace_bytes(mode, n, k, rows), dtype=torch.uint8, device="cuda")
        y = q8.matmul_rows_ws(mode, w, n, k, residual=resd, workspace=ws, **act)
        y2 = q8.matmul_rows_ws(mode, w, n, k, residual=resd, workspace=ws, **act)
        torch.cuda.synchronize()
        assert torch.equal(y, y2)
        assert _counters_zero(ws, n)
        r, a = _expected(mode, blocks, n, k, x, res)
        gate(y.cpu().numpy(), r, a, f"k split random {n}x{k} rows={rows} {mode}")
