"""Parity of the HIP path with the CPU oracle, through the C ABI, on the GPU.

Both sides start from the same seeded f32 inputs (synth) and run the whole
path on their own: Q8_0 weight quantization, activation quantization, the
projection.  Quantized bytes and int32 block sums must match bit for bit; f32
outputs must pass the gate of helpers.gate.  Every workload call is run at its
full size.
"""
import random

import numpy as np
import pytest
import torch

import oracle
import q8_projection_amd as q8
import synth
from synth import workloads

from helpers import acts_of, gate, say, weights_of

pytestmark = pytest.mark.gpu

CALLS = workloads.all_calls()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    torch.cuda.set_device(0)
    q8.lib()
    yield


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_path(call, w_blocks_dev, x, residual=None, mode=None, out=None):
    """GPU quantize (integer modes) and project; returns (y, hi, lo, scale) on host."""
    mode = mode or call.mode
    xd = to_dev(x)
    res = None if residual is None else to_dev(residual)
    hi = lo = sc = None
    if mode == "f32":
        y = q8.matmul_rows(mode, w_blocks_dev, call.n, call.k, x=xd, residual=res, out=out)
    else:
        hi, lo, sc = q8.quantize_act(mode, xd)
        y = q8.matmul_rows(mode, w_blocks_dev, call.n, call.k, hi=hi, lo=lo, scale=sc, residual=res, out=out)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.cpu().numpy()
    return cpu(y), cpu(hi), cpu(lo), cpu(sc)


def oracle_path(call, blocks, x, residual=None, mode=None):
    mode = mode or call.mode
    if mode == "f32":
        return oracle.project(mode, blocks, call.n, call.k, x.shape[0], x=x, residual=residual), None
    hi, lo, sc = oracle.quantize_act(mode, x)
    return oracle.project(mode, blocks, call.n, call.k, x.shape[0], hi=hi, lo=lo, scale=sc,
                          residual=residual), (hi, lo, sc)


# ------------------------------------------------------------ weight quantization

def _distinct_weights():
    seen, out = set(), []
    for c in CALLS:
        key = (c.n, c.k, c.w_seed)
        if key not in seen:
            seen.add(key)
            out.append(c)
    return out


@pytest.mark.parametrize("call", _distinct_weights(), ids=lambda c: f"{c.name}_w{c.w_seed}")
def test_quantize_weights_bitwise(call):
    say("quantize_weights", call.name, call.n, call.k, call.w_seed)
    w, blocks = weights_of(call)
    got = q8.quantize_weights(to_dev(w))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), blocks)


@pytest.mark.parametrize("n,k,seed", [(1, 64, 40), (3, 192, 41), (37, 320, 42), (5, 2112, 43), (129, 4160, 44)])
def test_quantize_weights_ragged(n, k, seed):
    say("quantize_weights ragged", n, k, seed)
    w = synth.weights(n, k, seed, outlier_frac=0.1)
    w[0, :32] = 0.0                                     # an all-zero block
    w[-1, -32:] *= np.float32(1e-6)                     # a block with a binary16-subnormal scale
    got = q8.quantize_weights(to_dev(w))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.quantize_weights(w))


# -------------------------------------------------------- activation quantization

@pytest.mark.parametrize("call", [c for c in CALLS if c.mode != "f32"], ids=lambda c: c.name)
def test_quantize_act_bitwise(call):
    say("quantize_act", call.name, call.mode, call.rows, call.k)
    x = acts_of(call)
    hi, lo, sc = q8.quantize_act(call.mode, to_dev(x))
    torch.cuda.synchronize()
    ehi, elo, esc = oracle.quantize_act(call.mode, x)
    assert np.array_equal(hi.cpu().numpy(), ehi)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), esc.view(np.uint32))
    if call.mode == "i8x2":
        assert np.array_equal(lo.cpu().numpy(), elo)


def _edge_activation():
    """Blocks that exercise rounding ties, zero and tiny scales, and huge values."""
    x = synth.activations(3, 256, seed=77)
    x[0, :32] = 0.0                                          # zero block
    x[0, 32:64] = np.float32(3e-39) * synth.normal(78, 32)   # subnormal values and scale
    x[0, 64:96] = np.float32(2.0 ** -149)                    # scale underflows to zero
    x[1, :32] = np.arange(-16, 16, dtype=np.float32) + np.float32(0.5)   # exact ties at s = 1 ...
    x[1, 0] = np.float32(127.0)                                          # ... (max 127 gives s = 1)
    x[1, 32:64] = synth.normal(79, 32) * np.float32(1e30)     # huge values
    x[2, :32] = np.float32(-1.0)                               # constant block
    return x


@pytest.mark.parametrize("mode", ["i8", "i8x2"])
def test_quantize_act_edges(mode):
    say("quantize_act edges", mode)
    x = _edge_activation()
    hi, lo, sc = q8.quantize_act(mode, to_dev(x))
    torch.cuda.synchronize()
    ehi, elo, esc = oracle.quantize_act(mode, x)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), esc.view(np.uint32))
    assert np.array_equal(hi.cpu().numpy(), ehi)
    if mode == "i8x2":
        assert np.array_equal(lo.cpu().numpy(), elo)


# ------------------------------------------------------------------ projection

@pytest.mark.parametrize("call", CALLS, ids=lambda c: c.name)
def test_projection_parity(call):
    say("projection", call.name, call.entry, call.mode, f"rows={call.rows}", f"{call.n}x{call.k}")
    w, blocks = weights_of(call)
    wd = q8.quantize_weights(to_dev(w))
    x = acts_of(call)
    res = call.make_residual()
    y, hi, lo, sc = gpu_path(call, wd, x, res)
    (r, a), q = oracle_path(call, blocks, x, res)
    assert np.array_equal(wd.cpu().numpy(), blocks)
    if q is not None:
        assert np.array_equal(hi, q[0]) and np.array_equal(sc.view(np.uint32), q[2].view(np.uint32))
        if call.mode == "i8x2":
            assert np.array_equal(lo, q[1])
    rel, ulps = gate(y, r, a, call.name)
    say("projection", call.name, f"max rel err {rel:.3g}", f"max ulps {ulps}")


def test_matvec_entry_point():
    """q8_matvec is the rows == 1 projection: same bits as q8_matmul_rows."""
    call = workloads.attn()[0]
    say("matvec entry", call.name)
    w, blocks = weights_of(call)
    wd = to_dev(blocks)
    x = acts_of(call)
    res = to_dev(call.make_residual())
    hi, lo, sc = q8.quantize_act(call.mode, to_dev(x))
    y1 = q8.matvec(call.mode, wd, call.n, call.k, hi=hi[0], lo=lo[0], scale=sc[0], residual=res[0])
    y2 = q8.matmul_rows(call.mode, wd, call.n, call.k, hi=hi, lo=lo, scale=sc, residual=res)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2[0])


# ------------------------------------------------------------------ block sums

# q8_block_sums runs the kernel the projection of the same call dispatches to,
# with its block-sum export on: the GEMV LDS ring (rows 1..2 and stacks the MFMA
# kernels do not take), the one-thread-per-block stand-in for the GEMV kernels
# without an export (k not a multiple of 256, or a stack staged in column
# tiles), the wave-private MFMA kernel (one activation tile on short matrices)
# and the shared-ring MFMA kernel in every (weight tiles, activation tiles)
# class, two-word and one-word (one-word stacks of up to 8 rows in the
# two-word layout), stacks over 64 rows (64-row slices), and the workload
# shapes at full size.
_SUMS_CASES = (
    [(256, 1024, 1, m) for m in ("i8", "i8x2")]
    + [(4096, 14336, 1, "i8x2"), (151936, 2048, 1, "i8"), (4096, 4096, 1, "i8x2")]   # GEMV ring, one row
    + [(9000, 1024, 2, "i8x2"), (9000, 1024, 2, "i8")]                              # GEMV ring, two rows
    + [(37, 2112, 3, "i8"), (13, 4160, 5, "i8x2"), (50, 4160, 8, "i8x2")]           # GEMV stand-in
    + [(300, 4096, 8, "i8x2"), (4096, 14336, 8, "i8x2"), (1000, 2304, 7, "i8"),     # wave-private MFMA
       (4000, 4096, 16, "i8"), (1, 256, 2, "i8x2"), (700, 2048, 2, "i8x2")]
    + [(n, 1024, rows, mode) for n in (2000, 6000, 9000)                              # shared-ring MFMA
       for rows, mode in ((5, "i8"), (24, "i8"), (64, "i8"), (5, "i8x2"), (12, "i8x2"), (24, "i8x2"),
                          (64, "i8x2"))]
    + [(14336, 4096, 8, "i8x2"), (14336, 4096, 64, "i8"), (14336, 4096, 2, "i8x2")]  # workload shapes
    + [(515, 4096, r, m) for r in (3, 9, 17, 33, 63) for m in ("i8", "i8x2")]        # ragged stacks
    + [(100, 512, 70, "i8x2"), (333, 768, 129, "i8")]                                 # over 64 rows
)


@pytest.mark.parametrize("n,k,rows,mode", _SUMS_CASES, ids=lambda v: str(v))
def test_block_sums_bitwise(n, k, rows, mode):
    say("block_sums", mode, n, k, rows)
    w = synth.weights(n, k, seed=90 + rows + n % 7, outlier_frac=0.01)
    x = synth.activations(rows, k, seed=95 + rows + k % 5, outlier_frac=0.005)
    blocks = oracle.quantize_weights(w)
    hi, lo, sc = oracle.quantize_act(mode, x)
    got = q8.block_sums(mode, to_dev(blocks), n, k, to_dev(hi), None if lo is None else to_dev(lo))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.block_sums(mode, blocks, n, k, hi, lo))


# ------------------------------------------------------------ ragged and edges

@pytest.mark.parametrize("mode", ["f32", "i8", "i8x2"])
@pytest.mark.parametrize("n,k,rows", [(1, 64, 1), (3, 192, 2), (7, 2112, 3), (13, 4160, 5), (37, 320, 8),
                                      (29, 1024, 9), (17, 512, 12), (11, 256, 64), (5, 128, 65),
                                      (130, 4096, 7), (1000, 1024, 2), (1000, 512, 17), (333, 768, 33),
                                      (20000, 256, 6), (64, 2048, 48), (257, 256, 63)])
def test_ragged_shapes(mode, n, k, rows):
    say("ragged", mode, n, k, rows)
    w = synth.weights(n, k, seed=200 + n, outlier_frac=0.1)
    x = synth.activations(rows, k, seed=300 + k, outlier_frac=0.05)
    res = synth.normal(400 + rows, (rows, n))
    blocks = oracle.quantize_weights(w)
    call = workloads.Call("ragged", n, k, rows, mode, "matmul_rows", w_seed=0)
    y, *_ = gpu_path(call, to_dev(blocks), x, res)
    (r, a), _ = oracle_path(call, blocks, x, res)
    gate(y, r, a, f"ragged {mode} {n}x{k} rows={rows}")


def _random_shapes(count, seed):
    """Seeded (n, k, rows, mode) draws over every dispatch path: k any multiple
    of 64 (the GEMV where it is not a multiple of 256), 1..70 rows, n from 1
    to 20000, each stack under 4096 x 14336 x 16 multiply-adds."""
    rng = random.Random(seed)
    out = []
    while len(out) < count:
        mode = rng.choice(["f32", "i8", "i8x2"])
        n = rng.choice([rng.randint(1, 300), rng.randint(300, 5000), rng.randint(5000, 20000)])
        k = 64 * rng.randint(1, 160)
        rows = rng.choice([rng.randint(1, 8), rng.randint(9, 70)])
        if n * k * rows <= 4096 * 14336 * 16:
            out.append((n, k, rows, mode))
    return out


def test_random_shapes():
    """24 seeded random shapes with outliers in weights and activations and a
    residual, through q8_matmul_rows, against the oracle."""
    for i, (n, k, rows, mode) in enumerate(_random_shapes(24, seed=777)):
        say("random", i, mode, n, k, rows)
        w = synth.weights(n, k, seed=7000 + i, outlier_frac=0.05)
        x = synth.activations(rows, k, seed=7100 + i, outlier_frac=0.05)
        res = synth.normal(7200 + i, (rows, n))
        blocks = oracle.quantize_weights(w)
        call = workloads.Call("random", n, k, rows, mode, "matmul_rows", w_seed=0)
        y, *_ = gpu_path(call, to_dev(blocks), x, res)
        (r, a), _ = oracle_path(call, blocks, x, res)
        gate(y, r, a, f"random {mode} {n}x{k} rows={rows}")


def test_stack_rows_equal_single_rows():
    """A row's result does not depend on the rest of its stack.  f32 mode (the
    GEMV family up to 4 rows): a stacked row equals that row alone.
    Integer modes, on a matrix short enough that a workgroup owns one 16-row
    weight tile: stacks of one activation tile (up to 8 two-word or 16 one-word
    rows) run on the wave-private MFMA kernel, taller ones on the shared-ring
    MFMA kernel.  Block terms are summed in f64 and each output is rounded once
    to f32, so where two stacks add the terms in different orders their f64
    totals differ by a few f64 ulps at most and the f32 outputs agree unless a
    total falls that close to an f32 rounding boundary (none does for this
    seeded input).  A row of an 8-row stack equals the same row in a 4-row
    stack, and a row of a 64-row stack the same row in a 24-row and in the
    8-row stack.  The GEMV on the row alone is within the gate."""
    n, k = 515, 4096
    say("stack vs single rows", n, k)
    w = synth.weights(n, k, seed=501)
    x64 = synth.activations(64, k, seed=502)
    blocks = oracle.quantize_weights(w)
    wd = to_dev(blocks)
    xd = to_dev(x64[:4])
    ys = q8.matmul_rows("f32", wd, n, k, x=xd)
    singles = [q8.matvec("f32", wd, n, k, x=xd[r]) for r in range(4)]
    torch.cuda.synchronize()
    for r in range(4):
        assert torch.equal(ys[r], singles[r]), ("f32", r)
    for mode in ("i8", "i8x2"):
        hi, lo, sc = q8.quantize_act(mode, to_dev(x64))

        def stack(r0, r1):
            return q8.matmul_rows(mode, wd, n, k, hi=hi[r0:r1], lo=None if lo is None else lo[r0:r1],
                                  scale=sc[r0:r1])

        ys64, ys24, ys8 = stack(0, 64), stack(0, 24), stack(0, 8)
        for r0 in range(0, 8, 4):
            ys4 = stack(r0, r0 + 4)
            torch.cuda.synchronize()
            assert torch.equal(ys8[r0:r0 + 4], ys4), (mode, r0)
        torch.cuda.synchronize()
        assert torch.equal(ys64[:24], ys24), mode
        assert torch.equal(ys64[:8], ys8), mode
        ohi, olo, osc = oracle.quantize_act(mode, x64)
        r, a = oracle.project(mode, blocks, n, k, 64, hi=ohi, lo=olo, scale=osc)
        gate(ys8.cpu().numpy(), r[:8], a[:8], f"stack of 8 {mode}")
        gate(ys64.cpu().numpy(), r, a, f"stack of 64 {mode}")
        one = q8.matvec(mode, wd, n, k, hi=hi[3], lo=None if lo is None else lo[3], scale=sc[3])
        torch.cuda.synchronize()
        gate(one.cpu().numpy(), r[3], a[3], f"single {mode}")


@pytest.mark.parametrize("mode", ["i8", "i8x2"])
@pytest.mark.parametrize("n,k,rows", [(5000, 2048, 1), (4096, 14336, 1), (700, 1088, 1), (1000, 4096, 3),
                                      (999, 2048, 8), (300, 512, 8), (4096, 4096, 1), (600, 8192, 8)])
def test_quantization_inside_the_projection_is_bitwise_the_same(mode, n, k, rows):
    """An integer-mode stack given as f32 x is quantized inside the projection
    (fused into its consumer) with the same bits as q8_quantize_act followed by
    the projection, whatever kernel runs it."""
    say("quantize inside", mode, n, k, rows)
    w = synth.weights(n, k, seed=1400 + n)
    x = synth.activations(rows, k, seed=1500 + k, outlier_frac=0.02)
    res = synth.normal(1600 + rows, (rows, n))
    wd = to_dev(oracle.quantize_weights(w))
    xd, rd = to_dev(x), to_dev(res)
    hi, lo, sc = q8.quantize_act(mode, xd)
    separate = q8.matmul_rows(mode, wd, n, k, hi=hi, lo=lo, scale=sc, residual=rd)
    inside = q8.matmul_rows(mode, wd, n, k, x=xd, residual=rd)
    gemv_separate = torch.cat([q8.matmul_rows(mode, wd, n, k, hi=hi[r0:r0 + 1],
                                              lo=None if lo is None else lo[r0:r0 + 1], scale=sc[r0:r0 + 1],
                                              residual=rd[r0:r0 + 1]) for r0 in range(rows)])
    inside_rows = torch.cat([q8.matmul_rows(mode, wd, n, k, x=xd[r0:r0 + 1], residual=rd[r0:r0 + 1])
                             for r0 in range(rows)])
    torch.cuda.synchronize()
    # one row at a time both run the GEMV: identical bits
    assert torch.equal(inside_rows, gemv_separate)
    # a stack: the fused call runs the GEMV in 8-row chunks, the separate one may
    # run the MFMA kernel (another summation order): both within the gate
    (r, a), _ = oracle_path(workloads.Call("q", n, k, rows, mode, "matmul_rows", w_seed=0),
                            oracle.quantize_weights(w), x, res)
    gate(inside.cpu().numpy(), r, a, f"inside {mode} {n}x{k} rows={rows}")
    gate(separate.cpu().numpy(), r, a, f"separate {mode} {n}x{k} rows={rows}")
    if rows <= 2:
        assert torch.equal(inside, separate)


@pytest.mark.parametrize("n,k,mode,with_res,inside", [(151936, 2048, "i8", False, False),
                                                     (50000, 4096, "i8x2", True, False),
                                                     (1000, 1088, "i8", False, False),
                                                     (3000, 2048, "f32", True, False),
                                                     (20000, 2048, "i8", False, True)])
def test_argmax_fused_into_the_projection(n, k, mode, with_res, inside):
    """One launch writes y and argmax y (the lowest index among equal maxima);
    y is bitwise the plain projection's, the index is the first maximum of that
    y, and the workspace's counter comes back to zero, ready for the next call."""
    say("argmax", n, k, mode, with_res, inside)
    w = synth.weights(n, k, seed=1700 + n % 97)
    x = synth.activations(1, k, seed=1800 + k)[0]
    res = synth.normal(1900, (n,)) if with_res else None
    wd, xd = to_dev(oracle.quantize_weights(w)), to_dev(x)
    rd = None if res is None else to_dev(res)
    if mode == "f32":
        args = dict(x=xd)
    elif inside:
        args = dict(x=xd)
    else:
        hi, lo, sc = q8.quantize_act(mode, xd.unsqueeze(0))
        args = dict(hi=hi[0], lo=None if lo is None else lo[0], scale=sc[0])
    y_ref = q8.matvec(mode, wd, n, k, residual=rd, **args)
    work = torch.zeros(q8.argmax_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    for call in range(2):
        y, idx = q8.matvec_argmax(mode, wd, n, k, residual=rd, workspace=work, **args)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), call
        y_np = y.cpu().numpy()
        assert int(idx.item()) == int(np.argmax(y_np)), call
        assert int(work[:16].count_nonzero().item()) == 0, call
    # the oracle agrees wherever its top two are further apart than the gate
    if mode == "f32":
        r, a = oracle.project(mode, oracle.quantize_weights(w), n, k, 1, x=x[None], residual=None if res is None else res[None])
    else:
        ohi, olo, osc = oracle.quantize_act(mode, x[None])
        r, a = oracle.project(mode, oracle.quantize_weights(w), n, k, 1, hi=ohi, lo=olo, scale=osc,
                              residual=None if res is None else res[None])
    gate(y_ref.cpu().numpy()[None], r, a, f"argmax head y {n}x{k} {mode}")
    r, a = r[0], a[0]
    top = np.argsort(r)[::-1][:2]
    tol = 1e-5 * abs(r[top]) + 2.0 ** -40 * a[top]
    if r[top[0]] - r[top[1]] > 2 * tol.max():
        assert int(idx.item()) == int(top[0])


@pytest.mark.parametrize("n,k,mode,calls", [(151936, 2048, "i8", 48), (20000, 1024, "i8x2", 96)])
def test_argmax_many_calls_in_a_row(n, k, mode, calls):
    """The arg-max's hand-off between workgroups (partials posted with
    agent-scope stores, an atomic arrival counter, the last workgroup reading
    the partials) over many launches queued back to back on one stream and one
    workspace, with no host synchronisation between them: each call projects a
    different activation row, so the maximum moves from call to call.  Every
    call's index must be the first maximum of its own y, every y the plain
    projection's, and the counter back at zero at the end.  Then the same
    sequence captured in a HIP graph and replayed three times."""
    say("argmax calls in a row", n, k, mode, calls)
    w = synth.weights(n, k, seed=2100 + n % 89)
    xs = synth.activations(calls, k, seed=2200 + calls, outlier_frac=0.01)
    wd = to_dev(oracle.quantize_weights(w))
    hi, lo, sc = q8.quantize_act(mode, to_dev(xs))
    work = torch.zeros(q8.argmax_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    ys = torch.empty((calls, n), dtype=torch.float32, device="cuda")
    idx = torch.full((calls,), -1, dtype=torch.int32, device="cuda")

    def run_all():
        for c in range(calls):
            q8.matvec_argmax(mode, wd, n, k, hi=hi[c], lo=None if lo is None else lo[c], scale=sc[c],
                             out=ys[c], idx=idx[c:c + 1], workspace=work)

    def check(tag):
        first_max = torch.argmax((ys == ys.max(dim=1, keepdim=True).values).to(torch.int32), dim=1)
        assert torch.equal(idx.to(torch.int64), first_max), tag
        assert int(work[:16].count_nonzero().item()) == 0, tag

    run_all()
    torch.cuda.synchronize()
    plain = torch.stack([q8.matvec(mode, wd, n, k, hi=hi[c], lo=None if lo is None else lo[c], scale=sc[c])
                         for c in range(calls)])
    torch.cuda.synchronize()
    assert torch.equal(ys, plain)
    check("eager")
    assert len(set(idx.tolist())) > 1  # the maximum does move between calls
    ref_idx = idx.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run_all()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        ys.zero_()
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, plain), rep
        assert torch.equal(idx, ref_idx), rep
        check(f"replay {rep}")


def test_argmax_ties_go_to_the_lowest_index():
    n, k = 4000, 2048
    say("argmax ties", n, k)
    w = synth.weights(n, k, seed=2001)
    x = synth.activations(1, k, seed=2002)
    xd = to_dev(x[0])
    hi, lo, sc = q8.quantize_act("i8", xd.unsqueeze(0))
    y = q8.matvec("i8", to_dev(oracle.quantize_weights(w)), n, k, hi=hi[0], scale=sc[0])
    torch.cuda.synchronize()
    m = int(torch.argmax(y).item())
    low, high = m // 3, min(n - 1, m + 17 if m + 17 < n else m - 1)
    w2 = w.copy()
    w2[low] = w[m]      # an exact copy of the maximum row below it ...
    w2[high] = w[m]     # ... and one above it
    wd2 = to_dev(oracle.quantize_weights(w2))
    y2, idx = q8.matvec_argmax("i8", wd2, n, k, hi=hi[0], scale=sc[0])
    torch.cuda.synchronize()
    assert float(y2[low]) == float(y2[m]) == float(y2[high]) == float(y2.max())
    assert int(idx.item()) == min(low, m, high)


def test_inplace_residual_and_adjacent_buffers():
    n, k, rows = 1000, 2048, 4
    say("in-place residual", n, k, rows)
    w = synth.weights(n, k, seed=601)
    x = synth.activations(rows, k, seed=602)
    res = synth.normal(603, (rows, n))
    wd = to_dev(oracle.quantize_weights(w))
    hi, lo, sc = q8.quantize_act("i8x2", to_dev(x))
    y_sep = q8.matmul_rows("i8x2", wd, n, k, hi=hi, lo=lo, scale=sc, residual=to_dev(res))
    buf = torch.empty(2 * rows * n, dtype=torch.float32, device="cuda")
    inplace = buf[:rows * n].view(rows, n)                      # y == residual, with y's
    inplace.copy_(to_dev(res))                                  # neighbour right after it
    q8.matmul_rows("i8x2", wd, n, k, hi=hi, lo=lo, scale=sc, residual=inplace, out=inplace)
    torch.cuda.synchronize()
    assert torch.equal(inplace, y_sep)


@pytest.mark.parametrize("n,k,rows", [(333, 1088, 6), (333, 1024, 6), (333, 1024, 40)])
def test_outputs_stay_in_bounds(n, k, rows):
    """Canary words around every output and quantized input are left untouched."""
    say("canaries", n, k, rows)
    w = synth.weights(n, k, seed=701)
    x = synth.activations(rows, k, seed=702)
    pad = 4096
    canary = -7.77e33
    wd = to_dev(oracle.quantize_weights(w))
    for mode in ("f32", "i8", "i8x2"):
        yb = torch.full((rows * n + 2 * pad,), canary, dtype=torch.float32, device="cuda")
        y = yb[pad:pad + rows * n].view(rows, n)
        xd = to_dev(x)
        if mode == "f32":
            q8.matmul_rows(mode, wd, n, k, x=xd, out=y)
        else:
            hb = torch.full((rows * k + 2 * pad,), 99, dtype=torch.int8, device="cuda")
            lb = torch.full((rows * k + 2 * pad,), 99, dtype=torch.int8, device="cuda")
            sb = torch.full((rows * (k // 32) + 2 * pad,), canary, dtype=torch.float32, device="cuda")
            hi = hb[pad:pad + rows * k].view(rows, k)
            lo = lb[pad:pad + rows * k].view(rows, k) if mode == "i8x2" else None
            sc = sb[pad:pad + rows * (k // 32)].view(rows, k // 32)
            q8.quantize_act(mode, xd, hi=hi, lo=lo, scale=sc)
            q8.matmul_rows(mode, wd, n, k, hi=hi, lo=lo, scale=sc, out=y)
            torch.cuda.synchronize()
            for t, c in ((hb, 99), (lb, 99)):
                assert (t[:pad] == c).all() and (t[-pad:] == c).all()
            assert (sb[:pad] == canary).all() and (sb[-pad:] == canary).all()
        torch.cuda.synchronize()
        assert (yb[:pad] == canary).all() and (yb[-pad:] == canary).all(), mode
        assert torch.isfinite(y).all()


def test_empty_problems_touch_nothing():
    say("empty problems")
    y = torch.full((4, 8), 3.0, device="cuda")
    wd = torch.zeros(8 * 34 * 2, dtype=torch.uint8, device="cuda")
    hi = torch.zeros((4, 64), dtype=torch.int8, device="cuda")
    sc = torch.zeros((4, 2), dtype=torch.float32, device="cuda")
    q8.matmul_rows("i8", wd, 8, 64, hi=hi, scale=sc, out=y, rows=0)
    q8.matmul_rows("i8", wd, 0, 64, hi=hi, scale=sc, out=y, rows=4)
    torch.cuda.synchronize()
    assert (y == 3.0).all()


def _hip():
    import ctypes
    h = ctypes.CDLL("libamdhip64.so")
    h.hipHostGetDevicePointer.restype = ctypes.c_int
    h.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    return h


def test_host_mapped_weights_same_bits():
    """Where the weight lives changes no value (codegen_cuda::lane page, Modules:
    residence): W in pinned host memory, read through the device address the
    runtime maps it to, gives the same bits as W in device memory."""
    import ctypes
    n, k = 257, 2048
    say("host-mapped weights", n, k)
    w = synth.weights(n, k, seed=801)
    x = synth.activations(2, k, seed=802)
    blocks = oracle.quantize_weights(w)
    w_dev = to_dev(blocks)
    w_host = torch.from_numpy(blocks).pin_memory()
    dptr = ctypes.c_void_p()
    if _hip().hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(w_host.data_ptr()), 0) != 0 or not dptr.value:
        pytest.skip("pinned host memory has no device mapping here")
    hi, lo, sc = q8.quantize_act("i8x2", to_dev(x))
    y_dev = q8.matmul_rows("i8x2", w_dev, n, k, hi=hi, lo=lo, scale=sc)
    y_host = torch.empty_like(y_dev)
    st = q8.lib().q8_matmul_rows(2, dptr, n, k, 2, ctypes.c_void_p(hi.data_ptr()), ctypes.c_void_p(lo.data_ptr()),
                                 ctypes.c_void_p(sc.data_ptr()), None, None, ctypes.c_void_p(y_host.data_ptr()),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(y_dev, y_host)


# Stacks of one activation tile (up to 8 two-word or 16 one-word rows): on a
# matrix short enough that a workgroup owns one 16-row weight tile they run on
# the wave-private MFMA kernel, else on the shared-ring one.  Cases: fewer
# chunks than waves, chunks that do not divide among the waves, a partial last
# tile, partial and empty row tiles of a workgroup owning 24 or 36 rows, full
# one-word tiles, one-word stacks of up to eight rows (run in the two-word
# layout), two- and three-row stacks, and the residual epilogue.
_WAVE_CASES = [(37, 256, 4, "i8x2", False), (1000, 2304, 7, "i8", True), (4000, 4096, 16, "i8", False),
               (100, 8192, 8, "i8x2", True), (4096, 1024, 5, "i8x2", True), (4001, 14336, 8, "i8x2", False),
               (9000, 4608, 8, "i8x2", True), (6000, 2048, 3, "i8", False), (14336, 4096, 6, "i8", True),
               (700, 2048, 2, "i8x2", True), (4096, 4096, 3, "i8x2", False), (2000, 1024, 3, "i8", True),
               (14336, 4096, 2, "i8x2", True), (9000, 1024, 2, "i8x2", False), (7000, 1024, 2, "i8x2", True),
               (4096, 4096, 2, "i8", True), (20000, 2048, 2, "i8", False), (14336, 2048, 8, "i8", True),
               (3000, 1024, 5, "i8", False), (1, 256, 2, "i8x2", True), (5, 256, 8, "i8", True)]


@pytest.mark.parametrize("n,k,rows,mode,with_res", _WAVE_CASES)
def test_mma_single_tile_kernels(n, k, rows, mode, with_res):
    say("mma single tile", n, k, rows, mode, with_res)
    w = synth.weights(n, k, seed=700 + n % 89)
    x = synth.activations(rows, k, seed=701 + rows)
    res = synth.normal(702, (rows, n)) if with_res else None
    blocks = oracle.quantize_weights(w)
    wd = to_dev(blocks)
    hi, lo, sc = q8.quantize_act(mode, to_dev(x))
    y = q8.matmul_rows(mode, wd, n, k, hi=hi, lo=lo, scale=sc, residual=None if res is None else to_dev(res))
    torch.cuda.synchronize()
    ohi, olo, osc = oracle.quantize_act(mode, x)
    r, a = oracle.project(mode, blocks, n, k, rows, hi=ohi, lo=olo, scale=osc, residual=res)
    gate(y.cpu().numpy(), r, a, f"mma single tile {n}x{k} rows={rows} {mode}")


# Every instantiation class of the MFMA kernel: a workgroup owns up to 16, 32 or
# 64 weight rows (n over the chip's 256 CUs: 2000, 6000, 9000) and the stack
# fills 1, 2, 4 or 8 activation tiles (16 columns each; two-word rows take two).
_MMA_CASES = [(n, rows, mode) for n in (2000, 6000, 9000)
              for rows, mode in ((5, "i8"), (24, "i8"), (64, "i8"),
                                 (5, "i8x2"), (12, "i8x2"), (24, "i8x2"), (64, "i8x2"))]


@pytest.mark.parametrize("n,rows,mode", _MMA_CASES)
def test_mma_instantiations(n, rows, mode):
    k = 1024
    say("mma instantiation", n, k, rows, mode)
    w = synth.weights(n, k, seed=600 + n % 97)
    x = synth.activations(rows, k, seed=601 + rows)
    blocks = oracle.quantize_weights(w)
    wd = to_dev(blocks)
    hi, lo, sc = q8.quantize_act(mode, to_dev(x))
    y = q8.matmul_rows(mode, wd, n, k, hi=hi, lo=lo, scale=sc)
    torch.cuda.synchronize()
    ohi, olo, osc = oracle.quantize_act(mode, x)
    r, a = oracle.project(mode, blocks, n, k, rows, hi=ohi, lo=olo, scale=osc)
    gate(y.cpu().numpy(), r, a, f"mma {n}x{k} rows={rows} {mode}")


@pytest.mark.parametrize("n,k,with_res", [(5000, 2304, True), (777, 6912, False), (3072, 4352, True),
                                          (100, 256, True), (14336, 6144, False), (50, 8192, True)])
def test_f32_row_on_both_grids(n, k, with_res):
    """The f32 mode at one row runs 12 waves a CU where three workgroups fit
    (k up to 6144, ragged k included), and the fused arg-max keeps the 8-wave
    grid.  Every row's total is one wave's, in the same order on either grid,
    so y is the same bits both ways; and it meets the oracle's gate."""
    say("f32 one row, both grids", n, k, with_res)
    w = synth.weights(n, k, seed=2100 + n % 89, outlier_frac=0.01)
    x = synth.activations(1, k, seed=2200 + k, outlier_frac=0.005)[0]
    res = synth.normal(2300, (n,)) if with_res else None
    blocks = oracle.quantize_weights(w)
    wd, xd = to_dev(blocks), to_dev(x)
    rd = None if res is None else to_dev(res)
    y = q8.matvec("f32", wd, n, k, x=xd, residual=rd)
    work = torch.zeros(q8.argmax_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    y8, _ = q8.matvec_argmax("f32", wd, n, k, x=xd, residual=rd, workspace=work)
    torch.cuda.synchronize()
    assert torch.equal(y, y8)
    r, a = oracle.project("f32", blocks, n, k, 1, x=x[None], residual=None if res is None else res[None])
    gate(y.cpu().numpy()[None], r, a, f"f32 {n}x{k}")


# ------------------------------------------------------------ weights over 1 GiB

_BIG_BLOCKS = {}


def _big_blocks():
    """A 32768x32768 Q8_0 matrix (1.06 GiB) of random bytes from a seeded
    generator: binary16 scales drawn around 1e-3, quants uniform in [-127, 127].
    Built once for the module."""
    if "b" not in _BIG_BLOCKS:
        n = k = 32768
        rng = np.random.default_rng(3100)
        nb = k // 32
        blocks = np.empty((n, nb, 34), dtype=np.uint8)
        scales = (np.abs(rng.standard_normal((n, nb))) * 1e-3 + 1e-4).astype(np.float16)
        blocks[:, :, 0:2] = scales.view(np.uint8).reshape(n, nb, 2)
        blocks[:, :, 2:] = rng.integers(-127, 128, size=(n, nb, 32), dtype=np.int8).view(np.uint8)
        _BIG_BLOCKS["b"] = blocks.reshape(n, nb * 34)
    return _BIG_BLOCKS["b"]


@pytest.mark.parametrize("mode,rows", [("i8x2", 9), ("i8", 16), ("i8x2", 1), ("i8", 2), ("f32", 1), ("f32", 5)])
def test_stacks_over_1gib_of_weights(mode, rows):
    """Weights of 1.06 GiB (32768x32768): every kernel family runs it as row
    slices of at most 1 GiB, one launch each (the int8 MFMA kernels: rows
    0..30831 and 30832..32767; the f64 MFMA kernel with two weight tiles a
    workgroup: 0..30815 and 30816..32767; the resident GEMV: 0..30839 and
    30840..32767; the tiled GEMV addresses each row group from its own base).  Outputs on both sides of the slice boundaries
    and at random places match the oracle one by one; in the integer modes the
    block sums of rows at the ends of the slices match it bit for bit."""
    n = k = 32768
    say("over 1 GiB", mode, rows, n, k)
    blocks = _big_blocks()
    rng = np.random.default_rng(3300 + rows)
    x = synth.activations(rows, k, seed=3200 + rows, outlier_frac=0.01)
    wd = to_dev(blocks)
    xd = to_dev(x)
    # slice ends: 30832 rows (int8 MFMA, multiples of 16), 30816 (f64 MFMA on
    # 32-row workgroups), 30840 (GEMV)
    edge_rows = np.array([0, 1, 30815, 30816, 30817, 30831, 30832, 30833, 30839, 30840, 30841, 32766, 32767])
    r_idx = np.concatenate([np.repeat(np.arange(rows), edge_rows.size), rng.integers(0, rows, 512)])
    n_idx = np.concatenate([np.tile(edge_rows, rows), rng.integers(0, n, 512)])
    if mode == "f32":
        y = q8.matmul_rows(mode, wd, n, k, x=xd)
        torch.cuda.synchronize()
        ry, ra = oracle.project_at(mode, blocks, n, k, rows, r_idx, n_idx, x=x)
    else:
        hi, lo, sc = q8.quantize_act(mode, xd)
        y = q8.matmul_rows(mode, wd, n, k, hi=hi, lo=lo, scale=sc)
        sums = q8.block_sums(mode, wd, n, k, hi, lo)
        torch.cuda.synchronize()
        ohi, olo, osc = oracle.quantize_act(mode, x)
        ry, ra = oracle.project_at(mode, blocks, n, k, rows, r_idx, n_idx, hi=ohi, lo=olo, scale=osc)
        want = oracle.block_sums(mode, blocks[edge_rows], edge_rows.size, k, ohi, olo)
        assert np.array_equal(sums[:, torch.from_numpy(edge_rows).cuda()].cpu().numpy(), want)
        del sums
    got = y.cpu().numpy()[r_idx, n_idx]
    gate(got[None], ry[None], ra[None], f"over 1 GiB {mode} rows={rows}")


# ------------------------------------------------------------ f32 stacks, f64 MFMA tiles

@pytest.mark.parametrize("n,k,rows,with_res", [(14336, 4096, 64, False), (4096, 14336, 16, True),
                                               (6144, 4096, 33, False), (4096, 4096, 9, True),
                                               (14336, 4096, 8, True), (4096, 14336, 5, False),
                                               (14336, 4096, 128, True), (8180, 1024, 16, True),
                                               (8176, 2048, 32, False), (8180, 1024, 24, True),
                                               (8180, 1024, 64, True), (8165, 2048, 48, False)])
def test_f32_stacks_at_full_size(n, k, rows, with_res):
    """f32 stacks of 5..64 rows (and two 64-row slices) at the workload shapes
    run on f64 MFMA tiles, every weight block read once a slice: all outputs
    against the oracle's gate.  A workgroup takes two weight tiles where that
    cuts the rounds of workgroups over the CUs enough: on 256 CUs the 6144-,
    8165..8180- and 14336-row cases here, not the 4096-row ones.  8180, 8176
    and 8165 rows end on a workgroup whose second tile is partly or wholly past
    the matrix, or whose first tile is short."""
    say("f32 stack", n, k, rows, with_res)
    w = synth.weights(n, k, seed=2400 + rows, outlier_frac=0.01)
    x = synth.activations(rows, k, seed=2500 + rows, outlier_frac=0.005, outlier_scale=20.0)
    res = synth.normal(2600 + rows, (rows, n)) if with_res else None
    blocks = oracle.quantize_weights(w)
    call = workloads.Call("f32_stack", n, k, rows, "f32", "matmul_rows", w_seed=0)
    y, *_ = gpu_path(call, to_dev(blocks), x, res)
    (r, a), _ = oracle_path(call, blocks, x, res)
    rel, ulps = gate(y, r, a, f"f32 stack {n}x{k} rows={rows}")
    say("f32 stack", f"max rel err {rel:.3g}", f"max ulps {ulps}")


@pytest.mark.parametrize("n,k,rows", [(37, 64, 9), (20, 128, 16), (300, 192, 33), (16, 64, 64), (1, 256, 5),
                                      (17, 320, 48)])
def test_f32_stacks_with_short_k(n, k, rows):
    """f32 stacks whose k gives fewer blocks than the f64 MFMA kernel has waves
    (k = 64: two blocks for eight waves), odd block counts per wave, and a
    weight tile with a single row or a ragged last tile."""
    say("f32 stack, short k", n, k, rows)
    w = synth.weights(n, k, seed=2900 + k, outlier_frac=0.05)
    x = synth.activations(rows, k, seed=2950 + rows, outlier_frac=0.05)
    res = synth.normal(2990, (rows, n))
    blocks = oracle.quantize_weights(w)
    call = workloads.Call("f32_short_k", n, k, rows, "f32", "matmul_rows", w_seed=0)
    y, *_ = gpu_path(call, to_dev(blocks), x, res)
    (r, a), _ = oracle_path(call, blocks, x, res)
    gate(y, r, a, f"f32 short k {n}x{k} rows={rows}")


@pytest.mark.parametrize("n", [515, 8180])
def test_f32_stack_rows_do_not_depend_on_the_stack(n):
    """On the f64 MFMA kernel each output is one lane's f64 total over the
    blocks, in an order fixed by k alone (block sums from chained MFMAs, then
    the waves' partials in wave order), whatever the other rows of the stack
    hold, however many activation tiles it has and however many weight tiles
    a workgroup takes: a row comes out with the same bits from stacks of 5, 9,
    16, 17, 33 and 64 rows and from offset stacks.  At 8180 rows every stack
    runs two weight tiles a workgroup; its first 515 weight rows alone run one
    tile a workgroup and give the same bits."""
    k = 4096
    say("f32 stack rows vs stack", n, k)
    w = synth.weights(n, k, seed=2701)
    x = synth.activations(64, k, seed=2702)
    wd, xd = to_dev(oracle.quantize_weights(w)), to_dev(x)
    full = q8.matmul_rows("f32", wd, n, k, x=xd)
    parts = {(r0, r1): q8.matmul_rows("f32", wd, n, k, x=xd[r0:r1].contiguous())
             for r0, r1 in ((0, 5), (0, 9), (0, 16), (0, 17), (0, 33), (20, 64), (50, 64), (56, 64))}
    head = {rows: q8.matmul_rows("f32", wd[:515].contiguous(), 515, k, x=xd[:rows].contiguous())
            for rows in (5, 17, 64)} if n > 515 else {}
    torch.cuda.synchronize()
    for (r0, r1), y in parts.items():
        assert torch.equal(y, full[r0:r1]), (r0, r1)
    for rows, y in head.items():
        assert torch.equal(y, full[:rows, :515]), rows


@pytest.mark.parametrize("n,rows", [(1000, 20), (8180, 40)])
def test_f32_stack_inplace_residual(n, rows):
    """y may be the residual buffer itself, with one or two weight tiles a
    workgroup (8180 rows take two)."""
    k = 2048
    say("f32 stack in-place residual", n, k, rows)
    w = synth.weights(n, k, seed=2801)
    x = synth.activations(rows, k, seed=2802)
    res = synth.normal(2803, (rows, n))
    wd, xd = to_dev(oracle.quantize_weights(w)), to_dev(x)
    y_sep = q8.matmul_rows("f32", wd, n, k, x=xd, residual=to_dev(res))
    buf = torch.empty(2 * rows * n, dtype=torch.float32, device="cuda")
    inplace = buf[:rows * n].view(rows, n)
    inplace.copy_(to_dev(res))
    q8.matmul_rows("f32", wd, n, k, x=xd, residual=inplace, out=inplace)
    torch.cuda.synchronize()
    assert torch.equal(inplace, y_sep)
