"""q8_matvec_argmax_noalloc (the fused arg-max head with the library's own
fixed workspace) against q8_matvec_argmax (a caller's workspace), through the C
ABI: the same y bit for bit and the same index, on calls in a row that share
the library's array, each smaller than the one before."""
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


def test_noalloc_argmax_matches_the_workspace_entry_point():
    torch.cuda.set_device(0)
    cases = [(151936, 2048, "i8", False), (20000, 1024, "i8x2", True), (3000, 2048, "f32", True)]
    for n, k, mode, with_res in cases:
        say("noalloc argmax", n, k, mode, with_res)
        w = _dev(oracle.quantize_weights(synth.weights(n, k, seed=2400 + n % 97)))
        x = _dev(synth.activations(1, k, seed=2500 + k)[0])
        res = _dev(synth.normal(2600, (n,))) if with_res else None
        if mode == "f32":
            args = dict(x=x)
        else:
            hi, lo, sc = q8.quantize_act(mode, x.unsqueeze(0))
            args = dict(hi=hi[0], lo=None if lo is None else lo[0], scale=sc[0])
        work = torch.zeros(q8.argmax_workspace_bytes(n), dtype=torch.uint8, device="cuda")
        y_ws, idx_ws = q8.matvec_argmax(mode, w, n, k, residual=res, workspace=work, **args)
        y_na = torch.full((n,), float("nan"), device="cuda")
        idx_na = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        q8.matvec_argmax_noalloc(mode, w, n, k, residual=res, out=y_na, idx=idx_na, **args)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), (n, k, mode)
        assert int(idx_na.item()) == int(idx_ws.item()) == int(torch.nonzero(y_ws == y_ws.max())[0].item())
