"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and every argument check returns its named status before anything is
enqueued (no call here reaches the HIP runtime).

Pointers are plain integers: validation looks at addresses only.  Every call
here must fail a check: a call that passed validation would launch a kernel on
these fake addresses.  Calls that pass (adjacent buffers, y == residual) are
covered by the GPU tests with real memory.
"""
import ctypes
import os
import re

import pytest

import q8_projection_amd as q8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8.h")

OK, NULL, SHAPE, ALIGN, MODE, ALIAS = 0, 1, 2, 3, 4, 5
BASE = 0x7f0000000000        # fake, well-aligned device addresses
MB = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert names == sorted(["q8_quantize_weights", "q8_quantize_act", "q8_matvec", "q8_matmul_rows",
                            "q8_matmul_rows_ws", "q8_matmul_rows_workspace_bytes",
                            "q8_matvec_argmax", "q8_argmax_workspace_bytes", "q8_matvec_argmax_noalloc",
                            "q8_block_sums",
                            "q8_status_name", "q8_version"])


def test_library_exports_every_declared_symbol():
    lib = q8.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in q8.SIGNATURES
    assert q8.version() == 100


def test_status_names():
    assert [q8.status_name(i) for i in range(7)] == [q8.STATUS[i] for i in range(7)]
    assert q8.status_name(99) == "Q8_E_UNKNOWN"


def _mv(mode=2, w=BASE, n=64, k=256, hi=BASE + 16 * MB, lo=BASE + 32 * MB, scale=BASE + 48 * MB,
        x=None, residual=None, y=BASE + 64 * MB, stream=None):
    return q8.lib().q8_matvec(mode, w, n, k, hi, lo, scale, x, residual, y, stream)


def _mm(mode=2, w=BASE, n=64, k=256, rows=4, hi=BASE + 16 * MB, lo=BASE + 32 * MB,
        scale=BASE + 48 * MB, x=None, residual=None, y=BASE + 64 * MB):
    return q8.lib().q8_matmul_rows(mode, w, n, k, rows, hi, lo, scale, x, residual, y, None)


def test_empty_problems_enqueue_nothing():
    assert _mv(n=0) == OK
    assert _mm(rows=0) == OK
    assert _mm(n=0) == OK
    assert q8.lib().q8_quantize_act(2, BASE, 0, 256, BASE + MB, BASE + 2 * MB, BASE + 3 * MB, None) == OK
    assert q8.lib().q8_quantize_weights(BASE, 0, 256, BASE + MB, None) == OK
    assert q8.lib().q8_block_sums(1, BASE, 5, 256, 0, BASE + MB, None, BASE + 2 * MB, None) == OK


@pytest.mark.parametrize("k", [0, -64, 32, 96, 100, 1 << 25])
def test_bad_k(k):
    assert _mv(k=k) == SHAPE
    assert q8.lib().q8_quantize_act(1, BASE, 1, k, BASE + MB, None, BASE + 2 * MB, None) == SHAPE
    assert q8.lib().q8_quantize_weights(BASE, 4, k, BASE + 8 * MB, None) == SHAPE


def test_bad_sizes():
    assert _mv(n=-1) == SHAPE
    assert _mm(rows=-1) == SHAPE
    assert _mv(n=1 << 40) == SHAPE


def test_modes():
    assert _mv(mode=3) == MODE
    assert _mv(mode=-1) == MODE
    assert q8.lib().q8_quantize_act(0, BASE, 1, 256, BASE + MB, None, BASE + 2 * MB, None) == MODE
    assert q8.lib().q8_block_sums(0, BASE, 4, 256, 1, BASE + MB, None, BASE + 2 * MB, None) == MODE


def test_null_pointers():
    assert _mv(w=None) == NULL
    assert _mv(y=None) == NULL
    assert _mv(hi=None) == NULL
    assert _mv(scale=None) == NULL
    assert _mv(mode=2, lo=None) == NULL
    assert _mv(mode=0, hi=None, lo=None, scale=None, x=None) == NULL
    # integer modes: the quantized stack, or x alone; a partial set is an error
    assert _mv(mode=2, hi=None, lo=None, scale=None, x=None) == NULL
    assert _mv(mode=2, hi=None, x=BASE + 96 * MB) == NULL                  # lo and scale still given
    assert _mv(mode=1, hi=None, lo=None, x=BASE + 96 * MB) == NULL         # scale still given
    assert _mm(mode=1, hi=BASE + 16 * MB, lo=None, scale=None, x=BASE + 96 * MB) == NULL
    # block sums never quantize: hi is required
    assert q8.lib().q8_block_sums(1, BASE, 4, 256, 1, None, None, BASE + 2 * MB, None) == NULL
    assert q8.lib().q8_quantize_act(2, BASE, 1, 256, BASE + MB, None, BASE + 2 * MB, None) == NULL
    assert q8.lib().q8_quantize_act(1, None, 1, 256, BASE + MB, None, BASE + 2 * MB, None) == NULL
    assert q8.lib().q8_quantize_weights(None, 4, 256, BASE + MB, None) == NULL


def test_integer_stacks_quantized_inside_take_at_most_eight_rows():
    """x alone in an integer mode is quantized inside one GEMV pass of at most 8
    rows; a taller stack is refused before anything is enqueued (the caller
    quantizes it once and passes hi, lo, scale)."""
    for mode, lo in ((1, None), (2, None)):
        for rows in (9, 17, 64, 65, 1000):
            assert _mm(mode=mode, rows=rows, hi=None, lo=lo, scale=None, x=BASE + 96 * MB) == SHAPE
    # validation still comes first: a bad mode or alignment is named as such
    assert _mm(mode=3, rows=9, hi=None, lo=None, scale=None, x=BASE + 96 * MB) == MODE
    assert _mm(mode=1, rows=9, hi=None, lo=None, scale=None, x=BASE + 96 * MB + 4) == ALIGN


def test_alignment():
    assert _mv(w=BASE + 2) == ALIGN
    assert _mv(hi=BASE + 16 * MB + 4) == ALIGN
    assert _mv(lo=BASE + 32 * MB + 8) == ALIGN
    assert _mv(scale=BASE + 48 * MB + 2) == ALIGN
    assert _mv(y=BASE + 64 * MB + 1) == ALIGN
    assert _mv(residual=BASE + 80 * MB + 2) == ALIGN
    assert _mv(mode=0, hi=None, lo=None, scale=None, x=BASE + 96 * MB + 4) == ALIGN
    assert _mv(mode=2, hi=None, lo=None, scale=None, x=BASE + 96 * MB + 8) == ALIGN
    assert q8.lib().q8_quantize_act(1, BASE + 4, 1, 256, BASE + MB, None, BASE + 2 * MB, None) == ALIGN
    assert q8.lib().q8_quantize_weights(BASE + 2, 4, 256, BASE + MB, None) == ALIGN


def test_aliasing():
    n, k = 64, 256
    wbytes = n * (k // 32) * 34
    assert _mv(y=BASE + wbytes - 4) == ALIAS                    # y runs into W's last bytes
    assert _mv(y=BASE + 16 * MB + 64) == ALIAS                  # inside hi
    assert _mv(y=BASE + 32 * MB) == ALIAS                       # on lo
    assert _mv(y=BASE + 48 * MB + 4) == ALIAS                   # inside scale
    assert _mv(mode=0, hi=None, lo=None, scale=None, x=BASE + 64 * MB - 256) == ALIAS
    assert _mv(mode=1, hi=None, lo=None, scale=None, x=BASE + 64 * MB - 256) == ALIAS
    assert _mm(mode=2, hi=None, lo=None, scale=None, x=BASE + 64 * MB - 4 * 256) == ALIAS
    r = BASE + 80 * MB
    assert _mv(residual=r, y=r + 4) == ALIAS                    # partial overlap with residual
    assert q8.lib().q8_quantize_act(2, BASE, 1, 256, BASE + 512, BASE + 2048, BASE + 4096, None) == ALIAS
    assert q8.lib().q8_quantize_act(2, BASE, 1, 256, BASE + MB, BASE + MB + 128, BASE + 2 * MB, None) == ALIAS


def _ma(mode=1, w=BASE, n=64, k=256, hi=BASE + 16 * MB, lo=BASE + 32 * MB, scale=BASE + 48 * MB, x=None,
        residual=None, y=BASE + 64 * MB, idx=BASE + 72 * MB, work=BASE + 76 * MB):
    return q8.lib().q8_matvec_argmax(mode, w, n, k, hi, lo, scale, x, residual, y, idx, work, None)


def test_split_workspace_size():
    """Workspace of the K-split projection: 32-bit counters, one per 16-row tile
    of the tallest matrix that splits (16 rows per CU: 256 counters, 1024 bytes,
    on a 256-CU device), then the f64 partials of every split of every range:
    integer modes 4 tiles of 16 weight rows by the activation tiles' rows (8 per
    two-word tile, 16 per one-word tile); f32 mode 2 tiles of 16 weight rows by
    16 rows per activation tile.  The device count of CUs is 256 here (MI355X,
    and the value assumed with no device)."""
    f = q8.lib().q8_matmul_rows_workspace_bytes
    part = lambda tiles, rows_per_tile: 4 * 16 * tiles * rows_per_tile * 8
    # 4096 x 28672, 8 two-word rows: 64 ranges, K in 4 parts (64 x 8 > 256 CUs)
    assert f(2, 4096, 28672, 8) == 1024 + 64 * 4 * part(1, 8)
    # 9 two-word rows: two tiles
    assert f(2, 4096, 28672, 9) == 1024 + 64 * 4 * part(2, 8)
    # 16 one-word rows: one tile of 16; 17: two
    assert f(1, 4096, 28672, 16) == 1024 + 64 * 4 * part(1, 16)
    assert f(1, 4096, 28672, 17) == 1024 + 64 * 4 * part(2, 16)
    # one-word rows up to 8 run in the two-word layout; 8 x 57344 bytes of stack
    assert f(1, 4096, 57344, 8) == f(2, 4096, 28672, 8)
    # 1000 rows: 16 ranges, K in 8 parts (nb = 896 is a multiple of 64)
    assert f(2, 1000, 28672, 8) == 1024 + 16 * 8 * part(1, 8)
    # the down projection 4096 x 14336: 16 two-word rows (459 KB), 64 one-word
    # rows (917 KB, four tiles) and 64 two-word rows (eight tiles)
    assert f(2, 4096, 14336, 16) == 1024 + 64 * 4 * part(2, 8)
    assert f(1, 4096, 14336, 64) == 1024 + 64 * 4 * part(4, 16)
    assert f(2, 4096, 14336, 64) == 1024 + 64 * 4 * part(8, 8)
    # more than 64 rows: 64-row slices one after another, the widest one's size
    assert f(2, 4096, 14336, 100) == f(2, 4096, 14336, 64)
    assert f(2, 4096, 14336, 65) == f(2, 4096, 14336, 64)
    # one tile on a full chip: from 400 KB of stack (rows x k, twice in
    # two-word mode)
    assert f(2, 4096, 25600, 8) > 0 and f(2, 4096, 25600, 7) == 0
    assert f(1, 4096, 25600, 16) > 0 and f(1, 4096, 25600, 15) == 0
    # at most 8 rows per CU, split over at least half the CUs: any height from
    # 2 rows, given 7 chunks a workgroup (512 rows: 64 workgroups, too few)
    assert f(2, 2048, 14336, 2) == 1024 + 32 * 8 * part(1, 8)
    assert f(1, 1024, 14336, 3) == 1024 + 16 * 8 * part(1, 8)
    assert f(2, 512, 14336, 8) == 0 and f(2, 512, 14336, 9) == 1024 + 8 * 8 * part(2, 8)
    # no split: f32 mode, one row, tall matrix, one tile on a full chip under
    # 400 KB (the down projection at 8 two-word rows: 229 KB; 16 one-word rows),
    # fewer than 7 chunks a workgroup (4096 x 4096, 2048 x 4096), K not in
    # whole chunks per part, k not a multiple of 256, bad sizes
    for args in ((2, 4096, 28672, 1), (2, 14336, 2048, 8), (2, 4096, 14336, 8),
                 (1, 4096, 14336, 16), (2, 4096, 4096, 48), (2, 2048, 4096, 8), (1, 4096, 28672, 8),
                 (2, 4096, 25344, 16), (2, 4096, 28672 - 64, 8), (2, 0, 28672, 8), (2, 4096, 28672, 0),
                 (2, -1, 28672, 8), (2, 4096, 100, 8), (7, 4096, 28672, 8)):
        assert f(*args) == 0, args
    # f32 mode: two weight tiles a workgroup over 32-row ranges, on matrices of
    # at most 16 rows per CU, from 5 rows (the f64 matrix-core kernel's floor)
    f32part = lambda tiles: 2 * 16 * tiles * 16 * 8
    assert f(0, 4096, 8192, 16) == 1024 + 128 * 2 * f32part(1)
    assert f(0, 4096, 4096, 24) == 1024 + 128 * 2 * f32part(2)
    # (32 rows: two activation tiles; 64-row plans need 112 KiB of LDS, more
    # than the 64 KiB assumed with no device)
    assert f(0, 2048, 4096, 32) == 1024 + 64 * 4 * f32part(2)
    # (no split: under 5 rows, tall matrix, one activation tile on a full chip
    # with under 128 blocks a part, bad k)
    for args in ((0, 4096, 4096, 4), (0, 4096, 4096, 1), (0, 14336, 4096, 16), (0, 4096, 4096, 16),
                 (0, 4096, 100, 16)):
        assert f(*args) == 0, args


def _mws(mode=2, w=BASE, n=4096, k=28672, rows=8, hi=BASE + 128 * MB, lo=BASE + 129 * MB,
         scale=BASE + 130 * MB, x=None, residual=None, y=BASE + 131 * MB, work=BASE + 132 * MB, work_bytes=2 * MB):
    return q8.lib().q8_matmul_rows_ws(mode, w, n, k, rows, hi, lo, scale, x, residual, y, work, work_bytes, None)


def test_split_projection_validation():
    """4096 x 28672 with 8 two-word rows: weights 119 MiB from BASE, hi, lo,
    scales and y 1 MiB apart above them, the workspace at +132 MiB."""
    need = q8.lib().q8_matmul_rows_workspace_bytes(2, 4096, 28672, 8)
    assert need > 0
    assert _mws(work=None) == NULL
    assert _mws(work=BASE + 132 * MB + 8) == ALIGN
    assert _mws(work_bytes=need - 1) == SHAPE
    assert _mws(work=BASE + 131 * MB + 64 * 1024) == ALIAS        # inside y
    assert _mws(work=BASE + 100 * MB) == ALIAS                    # inside the weights
    assert _mws(work=BASE + 130 * MB + 4096) == ALIAS             # inside the scales
    assert _mws(residual=BASE + 132 * MB + 4096) == ALIAS         # residual inside the workspace
    # empty problems enqueue nothing and need no workspace
    assert _mws(n=0, work=None) == OK
    assert _mws(rows=0, work=None) == OK
    # the projection's own checks come first
    assert _mws(mode=5) == MODE
    assert _mws(k=100) == SHAPE
    assert _mws(hi=None) == NULL
    assert _mws(y=BASE + 131 * MB + 2) == ALIGN
    assert _mws(y=BASE + 128 * MB + 4096) == ALIAS                # y over hi


def test_split_projection_validation_f32():
    """The f32 mode through the workspace entry (4096 x 8192, 16 rows: weights
    from BASE, x 512 KiB at +64 MiB, y at +66 MiB, the workspace at +68 MiB)."""
    lib = q8.lib()
    need = lib.q8_matmul_rows_workspace_bytes(0, 4096, 8192, 16)
    assert need > 0

    def f(x=BASE + 64 * MB, y=BASE + 66 * MB, work=BASE + 68 * MB, work_bytes=need):
        return lib.q8_matmul_rows_ws(0, BASE, 4096, 8192, 16, None, None, None, x, None, y, work, work_bytes, None)

    assert f(work=None) == NULL
    assert f(work_bytes=need - 8) == SHAPE
    assert f(x=BASE + 64 * MB + 4) == ALIGN
    assert f(work=BASE + 64 * MB + 128 * 1024) == ALIAS               # over x
    assert f(work=BASE + 66 * MB + 64) == ALIAS                       # over y


def test_argmax_workspace_size():
    lib = q8.lib()
    assert lib.q8_argmax_workspace_bytes(0) == 0
    assert lib.q8_argmax_workspace_bytes(-5) == 0
    assert lib.q8_argmax_workspace_bytes(1 << 31) == 0
    sizes = [lib.q8_argmax_workspace_bytes(n) for n in (1, 4, 5, 100, 151936)]
    assert all(b >= 24 and (b - 16) % 8 == 0 for b in sizes)
    assert sizes == sorted(sizes)


def test_argmax_validation():
    assert _ma(idx=None) == NULL
    assert _ma(work=None) == NULL
    assert _ma(hi=None) == NULL                                   # lo/scale given: a partial set
    assert _ma(idx=BASE + 72 * MB + 2) == ALIGN
    assert _ma(work=BASE + 76 * MB + 8) == ALIGN
    assert _ma(n=0) == SHAPE                                      # an arg-max of nothing
    assert _ma(mode=2, k=40000) == SHAPE                          # stack beyond the resident LDS budget
    assert _ma(mode=0, hi=None, lo=None, scale=None, x=BASE + 96 * MB, k=16448) == SHAPE
    assert _ma(n=1 << 20, k=1 << 15) == SHAPE                     # weights over 1 GiB: not one launch
    assert _ma(idx=BASE + 64 * MB + 8) == ALIAS                   # idx inside y
    assert _ma(work=BASE + 16) == ALIAS                           # workspace over W
    assert _ma(idx=BASE + 76 * MB + 16) == ALIAS                  # idx inside the workspace
    assert _ma(mode=3) == MODE


@pytest.mark.parametrize("rows,n", [(1 << 40, 64), (1 << 62, 1), (64, 1 << 62), ((1 << 31) // 64 + 1, 64),
                                    (3, (1 << 31) // 3 + 1)])
def test_huge_sizes_are_rejected_before_any_product(rows, n):
    """Sizes whose products would overflow int64 (or exceed the limits) are
    refused by name, without forming rows * n first."""
    assert _mm(rows=rows, n=n) == SHAPE
    assert q8.lib().q8_block_sums(2, BASE, n, 256, rows, BASE + MB, BASE + 2 * MB, BASE + 3 * MB, None) == SHAPE
    if n > (1 << 31):  # one row: only n can be too large
        assert q8.lib().q8_matvec_argmax(1, BASE, n, 256, BASE + MB, None, BASE + 2 * MB, None, None,
                                         BASE + 3 * MB, BASE + 4 * MB, BASE + 5 * MB, None) == SHAPE


def test_noalloc_argmax_refuses_what_its_array_cannot_hold():
    """q8_matvec_argmax_noalloc checks its arguments as q8_matvec_argmax does,
    and refuses a head whose partials would not fit its fixed 64 KiB array
    (every call here fails a check before anything is looked up or launched)."""
    f = q8.lib().q8_matvec_argmax_noalloc
    big = 5_000_000                       # 4.19 M rows is the most the array holds
    assert q8.lib().q8_argmax_workspace_bytes(big) > 65536
    assert f(1, BASE, big, 64, BASE + 512 * MB, None, BASE + 600 * MB, None, None, BASE + 700 * MB,
             BASE + 800 * MB, None) == SHAPE
    assert f(1, BASE, 64, 256, BASE + MB, None, BASE + 2 * MB, None, None, BASE + 3 * MB, None, None) == NULL
    assert f(1, BASE, 64, 256, BASE + MB, None, BASE + 2 * MB, None, None, BASE + 3 * MB, BASE + 4 * MB + 2,
             None) == ALIGN
    assert f(0, BASE, 64, 256, None, None, None, None, None, BASE + 3 * MB, BASE + 4 * MB, None) == NULL
    assert f(1, BASE, 64, 96, BASE + MB, None, BASE + 2 * MB, None, None, BASE + 3 * MB, BASE + 4 * MB,
             None) == SHAPE
    # idx inside y
    assert f(1, BASE, 64, 256, BASE + MB, None, BASE + 2 * MB, None, None, BASE + 3 * MB, BASE + 3 * MB + 8,
             None) == ALIAS
