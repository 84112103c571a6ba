"""The synthetic workloads of the Q8_0 projection: shapes, seeds and value
distributions of every call, shared by the tests and the benchmark.

Shapes follow the model forms on the pages: a decode step projects one row
(codegen_cuda::lane page, description), a batched decode step stacks one row per
sequence and a prefill chunk stacks the chunk's rows, with one pass over each
weight per stack; the LM head projects just the final row of a prefill chunk
(model::author page, Functions: decode_batch, prefill).

W is N x K (out x in).  Weights are N(0, 0.02^2), activations and residuals
N(0, 1).  Seeds are fixed; outlier rows/channels are picked on stream seed+1000.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import activations, normal, weights

MODES = ("f32", "i8", "i8x2")          # f32 + f64 sums | one-word int8 | two-word int8


@dataclass(frozen=True)
class Call:
    """One projection call of a workload."""
    name: str
    n: int
    k: int
    rows: int
    mode: str
    entry: str                               # "matvec" (rows == 1) or "matmul_rows"
    w_seed: int
    x_seed: int | None = None                # one stream for the whole stack
    x_row_seeds: tuple | None = None         # or one stream per row
    x_rows_total: int | None = None          # stack drawn with this many rows ...
    last_row_only: bool = False              # ... of which only the last is projected
    w_outlier_frac: float = 0.0
    w_outlier_scale: float = 8.0
    x_outlier_frac: float = 0.0
    x_outlier_scale: float = 20.0
    residual_seed: int | None = None
    tags: tuple = field(default_factory=tuple)

    @property
    def nb(self) -> int:
        return self.k // 32

    @property
    def weight_bytes(self) -> int:
        return self.n * self.nb * 34

    @property
    def flops(self) -> int:
        return 2 * self.rows * self.n * self.k

    def make_weights(self) -> np.ndarray:
        return weights(self.n, self.k, self.w_seed, 0.02, self.w_outlier_frac, self.w_outlier_scale)

    def make_activations(self) -> np.ndarray:
        """The activation rows this call projects, [rows][k] f32."""
        total = self.x_rows_total or self.rows
        if self.x_row_seeds is not None:
            x = activations(total, self.k, row_seeds=self.x_row_seeds,
                            outlier_frac=self.x_outlier_frac, outlier_scale=self.x_outlier_scale)
        else:
            x = activations(total, self.k, seed=self.x_seed,
                            outlier_frac=self.x_outlier_frac, outlier_scale=self.x_outlier_scale)
        if self.last_row_only:
            x = np.ascontiguousarray(x[-self.rows:])
        return x

    def make_residual(self) -> np.ndarray | None:
        if self.residual_seed is None:
            return None
        return normal(self.residual_seed, (self.rows, self.n))


def _modes(base: Call, modes=MODES):
    return [Call(**{**base.__dict__, "name": f"{base.name}_{m}", "mode": m}) for m in modes]


def tiny():
    """Tiny matvec: W 256x1024, one row, one-word int8."""
    return [Call("tiny", 256, 1024, 1, "i8", "matvec", w_seed=0, x_seed=1)]


def attn():
    """Decode attention projection: W 4096x4096 with 1% of rows x8, one activation row
    with 0.5% of channels x20, two-word int8, residual added."""
    return [Call("attn", 4096, 4096, 1, "i8x2", "matvec", w_seed=2, x_seed=3,
                 w_outlier_frac=0.01, w_outlier_scale=8.0,
                 x_outlier_frac=0.005, x_outlier_scale=20.0, residual_seed=4)]


def ffn():
    """Decode FFN at one row: up and gate 14336x4096, down 4096x14336, all three modes."""
    calls = []
    calls += _modes(Call("up", 14336, 4096, 1, "i8x2", "matvec", w_seed=5, x_seed=8))
    calls += _modes(Call("gate", 14336, 4096, 1, "i8x2", "matvec", w_seed=6, x_seed=8))
    calls += _modes(Call("down", 4096, 14336, 1, "i8x2", "matvec", w_seed=7, x_seed=9))
    return calls


def batched():
    """Batched decode, 8 rows with independent seeds, two-word: (i) 14336x4096;
    (ii) the down shape 4096x14336 with a residual 8x4096 added."""
    return [
        Call("batch8", 14336, 4096, 8, "i8x2", "matmul_rows", w_seed=10,
             x_row_seeds=tuple(range(11, 19))),
        Call("batch8_down_res", 4096, 14336, 8, "i8x2", "matmul_rows", w_seed=7,
             x_row_seeds=tuple(range(19, 27)), residual_seed=27),
    ]


def prefill():
    """Prefill chunk of 64 rows x 14336x4096 (one-word), then the LM head
    151936x2048 on the last row of a 64x2048 stack (one-word)."""
    return [
        Call("prefill64", 14336, 4096, 64, "i8", "matmul_rows", w_seed=28, x_seed=29),
        Call("lm_head", 151936, 2048, 1, "i8", "matvec", w_seed=30, x_seed=31,
             x_rows_total=64, last_row_only=True),
    ]


def decode_layer():
    """The projections of one decode layer at one row, two-word, in the order a
    decode step runs them (model::author page, Functions: decode_layer): fused
    QKV 6144x4096 (32 query heads and 8 key/value heads of 128 columns), O
    4096x4096 with the residual, gate and up 14336x4096 on one shared input,
    down 4096x14336 with the residual.  Not one of the parity workloads above:
    the graph test and the benchmark's decode-layer figure use it."""
    return [Call("layer_qkv", 6144, 4096, 1, "i8x2", "matvec", w_seed=40, x_seed=41),
            Call("layer_o", 4096, 4096, 1, "i8x2", "matvec", w_seed=42, x_seed=43, residual_seed=44),
            Call("layer_gate", 14336, 4096, 1, "i8x2", "matvec", w_seed=45, x_seed=46),
            Call("layer_up", 14336, 4096, 1, "i8x2", "matvec", w_seed=47, x_seed=46),
            Call("layer_down", 4096, 14336, 1, "i8x2", "matvec", w_seed=48, x_seed=49, residual_seed=50)]


WORKLOADS = {"tiny": tiny, "attn": attn, "ffn": ffn, "batched": batched, "prefill": prefill}


def all_calls():
    out = []
    for f in WORKLOADS.values():
        out += f()
    return out
