#!/usr/bin/env python3
"""Throughput of the Q8_0 projection hot path on one MI355X.

One step is one pass over every stage of the path, at the shapes the pages'
model forms run (codegen_cuda::lane page, description: decode steps, batched
decode, prefill chunks; model::author page, Functions: prefill, decode_batch):

  rows = 1   down projection   W 4096 x 14336, two-word   (quantize + q8_matvec)
  rows = 8   batched decode    W 14336 x 4096, two-word   (quantize + q8_matmul_rows)
  rows = 8   batched decode    W 4096 x 14336, two-word, residual epilogue
  rows = 64  prefill chunk     W 14336 x 4096, one-word   (quantize + q8_matmul_rows)
  rows = 1   LM head           W 151936 x 2048, one-word, the chunk's last row

Each call quantizes its activation rows on the GPU, then projects.  Weights are
synthetic (seeded, N(0, 0.02^2)), Q8_0-quantized on the GPU before timing and
resident in HBM.  Every matrix has two copies and consecutive steps alternate
between them.  A step then reads about 580 MB of distinct weights, so the 256 MB
Infinity Cache cannot serve a weight from the previous step.  The step is
captured in a HIP graph and replayed, as the lane replays each step
(codegen_cuda::lane page, description).

value = weight bytes of one step / step time (GB/s).  The JSON line also carries
per-call kernel times, the rows=1/8/64 bandwidths, the roofline of the dominant
kernel and the CPU oracle's throughput on a sample of the same work.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "Q8_0 projection effective weight GB/s and % HBM peak at rows=1/8/64"
PROFILES = os.path.join(ROOT, "profiles")


# Calls whose activation quantization runs inside the projection kernel (the
# stack passed as f32 x).  The tiny 256x1024 matvec is latency-bound, and the
# fused call takes 3.6 us against 5.2 us for a quantize launch plus the
# projection.  For the LM head the two are within noise (52.0 against
# 51.9-53.6 us), and the two-word calls lose (two correctly rounded divisions
# per value in every workgroup), so the step's calls quantize separately.
QUANTIZE_INSIDE: set = {"tiny"}


def step_calls():
    from synth import workloads as wl
    by_name = {c.name: c for c in wl.all_calls()}
    return [by_name["down_i8x2"], by_name["batch8"], by_name["batch8_down_res"], by_name["prefill64"],
            by_name["lm_head"]]


def other_calls():
    """The remaining configurations, timed per call outside the step: the tiny
    matvec (latency), the attention projection with its residual, and the
    rows=1 FFN shapes in all three activation modes."""
    from synth import workloads as wl
    by_name = {c.name: c for c in wl.all_calls()}
    return [by_name[n] for n in ("tiny", "attn", "up_f32", "up_i8", "up_i8x2", "down_f32", "down_i8", "down_i8x2")]


def kernel_hash(sources) -> str:
    """First 16 hex digits of the SHA-256 over the named kernel sources, in order."""
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(call_name: str):
    """HBM bytes per launch of a call from its committed counter summary (the
    profiles/*counters.txt whose `call` field names it), or None if there is none
    or it was taken on kernel sources other than the current ones."""
    try:
        for fname in sorted(os.listdir(PROFILES)):
            if not fname.endswith("counters.txt"):
                continue
            fields = {}
            with open(os.path.join(PROFILES, fname)) as f:
                for line in f:
                    if "=" in line and not line.lstrip().startswith("#"):
                        k, v = line.split("=", 1)
                        fields[k.strip()] = v.strip()
            if fields.get("call") != call_name:
                continue
            sources = fields.get("kernel_sources", "").split()
            if sources and fields.get("kernel_sources_sha256_16") == kernel_hash(sources):
                return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        pass
    return None


class Prepared:
    """Device buffers of one call: weight copies, activations, outputs."""

    def __init__(self, call, dev):
        import numpy as np
        import torch
        import q8_projection_amd as q8
        self.call = call
        # enough copies that cycling through them reads over 512 MiB between
        # two uses of one copy: none can be served from the Infinity Cache
        self.copies = max(2, -(-(512 << 20) // call.weight_bytes))
        w = torch.from_numpy(call.make_weights()).to(dev)
        self.w = [q8.quantize_weights(w) for _ in range(self.copies)]
        del w
        x = call.make_activations()
        self.x = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        res = call.make_residual()
        self.res = None if res is None else torch.from_numpy(res).to(dev)
        rows, k, n = call.rows, call.k, call.n
        self.hi = torch.empty((rows, k), dtype=torch.int8, device=dev)
        self.lo = torch.empty((rows, k), dtype=torch.int8, device=dev) if call.mode == "i8x2" else None
        self.sc = torch.empty((rows, k // 32), dtype=torch.float32, device=dev)
        self.y = torch.empty((rows, n), dtype=torch.float32, device=dev)

    @property
    def inside(self) -> bool:
        return self.call.name in QUANTIZE_INSIDE

    def quantize(self):
        import q8_projection_amd as q8
        if not self.inside and self.call.mode != "f32":
            q8.quantize_act(self.call.mode, self.x, hi=self.hi, lo=self.lo, scale=self.sc)

    def project(self, copy):
        import q8_projection_amd as q8
        c = self.call
        if c.mode == "f32":
            q8.matmul_rows(c.mode, self.w[copy], c.n, c.k, x=self.x, residual=self.res, out=self.y)
        elif self.inside:
            q8.matmul_rows(c.mode, self.w[copy], c.n, c.k, x=self.x,
                           residual=self.res, out=self.y)
        elif c.rows == 1:
            q8.matvec(c.mode, self.w[copy], c.n, c.k, hi=self.hi[0], lo=None if self.lo is None else self.lo[0],
                      scale=self.sc[0], residual=None if self.res is None else self.res[0], out=self.y[0])
        else:
            q8.matmul_rows(c.mode, self.w[copy], c.n, c.k, hi=self.hi, lo=self.lo, scale=self.sc,
                           residual=self.res, out=self.y)


def sweep(spec: str, dev, only_rows: int | None = None, launches: int = 0, ws: bool = False):
    """Kernel time of one projection per stack height (rows 1..64) through the
    library's own dispatch: "N,K,MODE", e.g. "14336,4096,i8x2".  Prints one JSON
    line per height.  With `only_rows`: run that height alone, eagerly,
    `launches` times (for profilers), and print one line.  With `ws`: call
    matmul_rows_ws with one zero-filled workspace for every height (the K split
    where the library splits, matmul_rows elsewhere; `split` says which)."""
    import dataclasses
    import torch
    import q8_projection_amd as q8
    from synth import workloads as wl
    n, k, mode = spec.split(",")
    base = wl.Call(f"sweep_{n}x{k}_{mode}", int(n), int(k), 64, mode, "matmul_rows", w_seed=900, x_seed=901)
    p = Prepared(base, dev)
    p.quantize()
    need = {r: q8.matmul_rows_workspace_bytes(mode, base.n, base.k, r) if ws else 0 for r in range(1, 65)}
    work = torch.zeros(max(16, *need.values()), dtype=torch.uint8, device=dev) if ws else None

    def launch(i, rows):
        if ws:
            lo = None if p.lo is None else p.lo[:rows]
            act = ({"x": p.x[:rows]} if mode == "f32" else
                   {"hi": p.hi[:rows], "lo": lo, "scale": p.sc[:rows]})
            q8.matmul_rows_ws(mode, p.w[i % p.copies], base.n, base.k, out=p.y[:rows], workspace=work, **act)
        elif mode == "f32":
            q8.matmul_rows(mode, p.w[i % p.copies], base.n, base.k, x=p.x[:rows], out=p.y[:rows])
        else:
            lo = None if p.lo is None else p.lo[:rows]
            q8.matmul_rows(mode, p.w[i % p.copies], base.n, base.k, hi=p.hi[:rows], lo=lo, scale=p.sc[:rows],
                           out=p.y[:rows])

    if only_rows is not None:
        if not 1 <= only_rows <= 64:
            raise ValueError("--rows: 1..64")
        torch.cuda.synchronize()
        for i in range(launches):
            launch(i, only_rows)
        torch.cuda.synchronize()
        call = dataclasses.replace(base, rows=only_rows)
        line = {"sweep": f"{n}x{k}", "mode": mode, "rows": only_rows, "launches": launches,
                "weight_bytes_per_launch": call.weight_bytes}
        if ws:
            line.update(entry="matmul_rows_ws", split=need[only_rows] > 0)
        print(json.dumps(line), flush=True)
        return
    for rows in (1, 2, 3, 4, 6, 8, 9, 12, 16, 24, 32, 48, 64):
        call = dataclasses.replace(base, rows=rows)
        reps = 20
        g = capture(lambda rows=rows: [launch(i, rows) for i in range(reps)])
        t = time_graph(g, 5) / reps
        line = {"sweep": f"{n}x{k}", "mode": mode, "rows": rows, "project_us": round(t * 1e6, 3),
                "GBps": round(call.weight_bytes / t / 1e9, 1),
                "pct_hbm_peak": round(call.weight_bytes / t / 1e9 / HBM_PEAK_GBPS * 100, 1),
                "rows_GFLOPs": round(call.flops / t / 1e9, 1)}
        if ws:
            line.update(entry="matmul_rows_ws", split=need[rows] > 0)
        print(json.dumps(line), flush=True)


def calib_copies(mib: int, dev) -> int:
    """torch's device copy of `mib` MiB, four times: the known-size reference
    that HBM byte counters are scaled by.  Returns the bytes of one copy."""
    import torch
    if not mib:
        return 0
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    return n


def time_calls(prepared, reps):
    """Per call: projection (and separate quantization) time from graphs of
    `reps` back-to-back launches on rotating weight copies."""
    out = {}
    for p in prepared:
        p.quantize()
        separate = not p.inside and p.call.mode != "f32"
        gq = capture(lambda p=p: p.quantize(), reps) if separate else None
        gp = capture(lambda p=p: [p.project(i % p.copies) for i in range(reps)])
        tq = 0.0 if gq is None else time_graph(gq, 5) / reps
        tp = time_graph(gp, 5) / reps
        out[p.call.name] = {"rows": p.call.rows, "n": p.call.n, "k": p.call.k, "mode": p.call.mode,
                            "weight_bytes": p.call.weight_bytes,
                            "project_us": round(tp * 1e6, 3),
                            "quantize_us": round(tq * 1e6, 3) if separate else None,
                            "quantize_inside": p.inside,
                            "GBps": round(p.call.weight_bytes / tp / 1e9, 1),
                            "pct_hbm_peak": round(p.call.weight_bytes / tp / 1e9 / HBM_PEAK_GBPS * 100, 1),
                            "rows_GFLOPs": round(p.call.flops / tp / 1e9, 1),
                            "hbm_bytes_counted": stored_traffic(p.call.name)}
    return out


def time_head_argmax(p, reps):
    """Kernel time of the LM head with its arg-max fused in (not part of the
    step); checks the index against the first maximum of the plain head's y."""
    import torch
    import q8_projection_amd as q8
    c = p.call
    p.quantize()
    p.project(0)
    torch.cuda.synchronize()
    y = p.y[0].clone()
    idx = torch.empty((1,), dtype=torch.int32, device=y.device)
    work = torch.zeros(q8.argmax_workspace_bytes(c.n), dtype=torch.uint8, device=y.device)
    out = torch.empty_like(y)

    # the same activation input as the plain head: the f32 row when its
    # quantization runs inside the projection, else the quantized row
    act = (dict(x=p.x[0]) if p.inside else
           dict(hi=p.hi[0], lo=None if p.lo is None else p.lo[0], scale=p.sc[0]))

    def launch(i):
        q8.matvec_argmax(c.mode, p.w[i % p.copies], c.n, c.k, out=out, idx=idx, workspace=work, **act)

    g = capture(lambda: [launch(i) for i in range(reps)])
    t = time_graph(g, 5) / reps
    want = int(torch.nonzero(y == y.max())[0].item())
    if not torch.equal(out, y) or int(idx.item()) != want:
        raise RuntimeError("the LM head with a fused arg-max differs from the plain head")
    return {"project_us": round(t * 1e6, 3), "GBps": round(c.weight_bytes / t / 1e9, 1),
            "pct_hbm_peak": round(c.weight_bytes / t / 1e9 / HBM_PEAK_GBPS * 100, 1), "index": want}


def decode_layer_calls():
    """The projections of one decode layer (synth.workloads.decode_layer)."""
    from synth import workloads as wl
    return wl.decode_layer()


def time_decode_layer(dev, iters, inside=False):
    """One decode layer's projections (decode_layer_calls), each input quantized
    once (gate and up share theirs): nine kernels a layer.  With `inside`, the
    projections of 4096-column inputs take the f32 input and quantize it in
    their own staging (six kernels).  Timed eagerly and as a replayed HIP
    graph, alternating two copies of every matrix (463 MB, more than the
    Infinity Cache); every replay must equal the eager layer."""
    import torch
    import q8_projection_amd as q8
    calls = decode_layer_calls()
    copies = 2
    wts = []
    for c in calls:
        w = torch.from_numpy(c.make_weights()).to(dev)
        wts.append([q8.quantize_weights(w) for _ in range(copies)])
        del w
    inputs = {}
    for c in calls:
        if c.x_seed not in inputs:
            x = torch.from_numpy(c.make_activations()).to(dev)
            inputs[c.x_seed] = (x, torch.empty((1, c.k), dtype=torch.int8, device=dev),
                                torch.empty((1, c.k), dtype=torch.int8, device=dev),
                                torch.empty((1, c.k // 32), dtype=torch.float32, device=dev))
    res = [None if c.residual_seed is None else torch.from_numpy(c.make_residual()).to(dev) for c in calls]
    ys = [torch.empty((1, c.n), dtype=torch.float32, device=dev) for c in calls]

    def layer(copy):
        done = set()
        for i, c in enumerate(calls):
            x, hi, lo, sc = inputs[c.x_seed]
            if inside and c.k <= 4096:
                q8.matvec("i8x2", wts[i][copy], c.n, c.k, x=x[0],
                          residual=None if res[i] is None else res[i][0], out=ys[i][0])
                continue
            if c.x_seed not in done:
                q8.quantize_act("i8x2", x, hi=hi, lo=lo, scale=sc)
                done.add(c.x_seed)
            q8.matvec("i8x2", wts[i][copy], c.n, c.k, hi=hi[0], lo=lo[0], scale=sc[0],
                      residual=None if res[i] is None else res[i][0], out=ys[i][0])

    layer(0)
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(4):
        layer(i % copies)
    e0.record(s)
    for i in range(iters):
        layer(i % copies)
    e1.record(s)
    e1.synchronize()
    eager = e0.elapsed_time(e1) / iters * 1e-3
    graphs = [capture(lambda c=c: layer(c)) for c in range(copies)]
    for g in graphs:
        for y in ys:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(y, r) for y, r in zip(ys, ref)):
            raise RuntimeError("decode-layer graph replay differs from the eager layer")
    for i in range(4):
        graphs[i % copies].replay()
    e0.record(s)
    for i in range(iters):
        graphs[i % copies].replay()
    e1.record(s)
    e1.synchronize()
    graph = e0.elapsed_time(e1) / iters * 1e-3
    nbytes = sum(c.weight_bytes for c in calls)
    return {"calls": [f"{c.name.split('_')[1]} {c.n}x{c.k}" + (" +res" if c.residual_seed is not None else "")
                      for c in calls],
            "kernels": 6 if inside else 9, "quantize_inside": inside, "weight_bytes": nbytes,
            "eager_us": round(eager * 1e6, 2),
            "graph_us": round(graph * 1e6, 2), "GBps_graph": round(nbytes / graph / 1e9, 1),
            "pct_hbm_peak_graph": round(nbytes / graph / 1e9 / HBM_PEAK_GBPS * 100, 1)}


def rows_summary(per_call, ceiling):
    """The metric's rows=1/8/64 figures, each on its own shapes: rows=1 is the
    4096x14336 down projection alone (the LM head, also one row, has an entry
    of its own), rows=8 the two batched calls together, rows=64 the prefill."""
    groups = {"1": ["down_i8x2"], "8": ["batch8", "batch8_down_res"], "64": ["prefill64"],
              "lm_head": ["lm_head"]}
    out = {}
    for key, names in groups.items():
        nbytes = sum(per_call[n]["weight_bytes"] for n in names)
        us = sum(per_call[n]["project_us"] for n in names)
        ceil_us = sum(ceiling[str(per_call[n]["weight_bytes"])]["us"] for n in names)
        gbps = nbytes / us / 1e3
        out[key] = {"calls": names, "GBps": round(gbps, 1), "pct_hbm_peak": round(gbps / HBM_PEAK_GBPS * 100, 1),
                    "pct_of_stream_ceiling": round(ceil_us / us * 100, 1)}
    return out


def capture(fn, reps=1):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the path on the capture stream once
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for _ in range(reps):
                fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def time_graph(g, iters):
    """Mean GPU time of one replay, from HIP events on the replay stream."""
    import torch
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(iters):
        g.replay()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters * 1e-3  # seconds


def stream_ceiling(sizes, dev, reps=20):
    """The measured streaming-read ceiling for each byte count: the bare read
    of libq8probe.so (no math, the GEMV's copy form and ring), over rotating
    buffers like the projections' weight copies, best over its ring depths
    (2, 4, 8 items a wave) and occupancies (4, 8, 16 waves a CU).  Time per
    launch from graphs of `reps` launches."""
    import ctypes
    import torch
    from q8_projection_amd import build as q8build
    if not os.path.exists(q8build.PROBE_LIB):
        raise ImportError(f"{q8build.PROBE_LIB} is missing: build it with q8_projection_amd/build.py")
    lib = ctypes.CDLL(q8build.PROBE_LIB)
    lib.q8probe_stream.restype = ctypes.c_int
    lib.q8probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    out = {}
    for size in sorted(set(sizes)):
        copies = max(2, -(-(512 << 20) // size))
        bufs = [torch.empty(size, dtype=torch.uint8, device=dev) for _ in range(copies)]
        best = None
        for ring in (2, 4, 8):
            for wpc in (4, 8, 16):
                def launch(i, ring=ring, wpc=wpc):
                    rc = lib.q8probe_stream(ctypes.c_void_p(bufs[i % copies].data_ptr()), size, ring, wpc,
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                    if rc != 0:
                        raise RuntimeError(f"q8probe_stream: {rc}")
                g = capture(lambda: [launch(i) for i in range(reps)])
                t = time_graph(g, 5) / reps
                if best is None or t < best[0]:
                    best = (t, ring, wpc)
        del bufs
        torch.cuda.empty_cache()
        t, ring, wpc = best
        out[str(size)] = {"us": round(t * 1e6, 3), "GBps": round(size / t / 1e9, 1),
                          "pct_hbm_peak": round(size / t / 1e9 / HBM_PEAK_GBPS * 100, 1),
                          "ring": ring, "waves_per_cu": wpc, "buffers": copies}
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(calls, budget_s: float):
    """The oracle on the host: activation quantization and projection of the same
    calls, on every 16th weight row (full K, all activation rows)."""
    import numpy as np
    import oracle
    import synth
    stride = 16
    work = []
    for c in calls:
        rows_sel = np.arange(0, c.n, stride)
        w = np.empty((rows_sel.size, c.k), dtype=np.float32)
        for i, r in enumerate(rows_sel):
            w[i] = synth.normal(c.w_seed, c.k, 0.02, offset=int(r) * c.k)
        if c.w_outlier_frac:
            raise ValueError("sampled weights do not model outlier rows")
        blocks = oracle.quantize_weights(w)
        x = c.make_activations()
        res = c.make_residual()
        res_s = None if res is None else np.ascontiguousarray(res[:, rows_sel])
        work.append((c, blocks, x, res_s, rows_sel.size))
    sample_bytes = sum(n_s * (c.k // 32) * 34 for c, _, _, _, n_s in work)

    def one_pass():
        for c, blocks, x, res_s, n_s in work:
            if c.mode == "f32":
                oracle.project(c.mode, blocks, n_s, c.k, x.shape[0], x=x, residual=res_s)
            else:
                hi, lo, sc = oracle.quantize_act(c.mode, x)
                oracle.project(c.mode, blocks, n_s, c.k, x.shape[0], hi=hi, lo=lo, scale=sc, residual=res_s)

    def timed(seconds, max_passes):
        one_pass()  # warm-up
        times = []
        t_end = time.perf_counter() + seconds
        while True:
            t0 = time.perf_counter()
            one_pass()
            times.append(time.perf_counter() - t0)
            if time.perf_counter() > t_end or len(times) >= max_passes:
                break
        return sorted(times)[len(times) // 2], len(times)

    all_threads = oracle.threads()
    med, n_all = timed(budget_s, 5000)
    oracle.set_threads(1)
    try:
        med1, n_one = timed(budget_s / 2, 500)
    finally:
        oracle.set_threads(all_threads)
    return {
        "value": round(sample_bytes / med / 1e9, 3),
        "unit": "GB/s",
        "cores": all_threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "value_1thread": round(sample_bytes / med1 / 1e9, 3),
        "sample": f"every {stride}th weight row of each call of the step (full K, all activation rows), "
                  f"{sample_bytes / 1e6:.1f} MB of Q8_0 weights; activation quantization + projection; "
                  f"median of {n_all} passes on {all_threads} threads (value) and of {n_one} passes on one "
                  f"thread (value_1thread), each after one warm-up pass",
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed step replays before the timed ones (200 steps are ~30 ms; with 10 the timed "
                         "steps ran about 1%% slower)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle timing on all threads (half as long again on one thread)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default=None, help="run only the named call eagerly (for profilers)")
    ap.add_argument("--sweep", default=None, metavar="N,K,MODE",
                    help="time one projection shape at stack heights 1..64 instead of the step")
    ap.add_argument("--rows", type=int, default=None,
                    help="with --sweep: run only this stack height, eagerly, warmup + steps launches (for profilers)")
    ap.add_argument("--ws", action="store_true",
                    help="with --sweep: call matmul_rows_ws (K split over workgroups where the library splits)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="with --only or --sweep --rows: also run torch's device copy of this many MiB, 4 times (the "
                         "known-size reference for HBM byte counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (a projection's share of a "
              "sharded layer is the same kernel at its own shape)", file=sys.stderr)
        return 2

    import torch
    import q8_projection_amd as q8

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    q8.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep:
        sweep(args.sweep, dev, args.rows, args.warmup + args.steps, ws=args.ws)
        if args.rows is not None and args.calib_copy_mib:
            print(json.dumps({"calib_copy_bytes_each": calib_copies(args.calib_copy_mib, dev)}))
        return 0
    if args.only:
        from synth import workloads as wl
        by_name = {c.name: c for c in wl.all_calls()}
        if args.only not in by_name:
            print(f"--only: no call named {args.only!r}; calls: {', '.join(by_name)}", file=sys.stderr)
            return 2
        p = Prepared(by_name[args.only], dev)
        torch.cuda.synchronize()
        p.quantize()
        for i in range(args.warmup + args.steps):
            p.project(i % p.copies)
        torch.cuda.synchronize()
        copied = calib_copies(args.calib_copy_mib, dev)
        print(json.dumps({"only": args.only, "launches": args.warmup + args.steps,
                          "weight_bytes_per_launch": p.call.weight_bytes, "calib_copy_bytes_each": copied}))
        return 0

    calls = step_calls()
    copies = 2  # the step graphs alternate two copies of every matrix
    prepared = [Prepared(c, dev) for c in calls]
    torch.cuda.synchronize()

    def step(copy):
        for p in prepared:
            p.quantize()
            p.project(copy)

    # eager reference outputs, then the graphs; every replay must reproduce them
    step(0)
    torch.cuda.synchronize()
    ref = [p.y.clone() for p in prepared]
    graphs = [capture(lambda c=c: step(c)) for c in range(copies)]
    for g in graphs:
        for p in prepared:
            p.y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for p, r in zip(prepared, ref):
            if not torch.equal(p.y, r):
                raise RuntimeError(f"graph replay differs from the eager step in {p.call.name}")

    for i in range(args.warmup):
        graphs[i % copies].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % copies].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_s = elapsed / args.steps
    step_bytes = sum(c.weight_bytes for c in calls)

    # per-call kernel times: a graph of back-to-back launches cycling the copies
    reps = 20
    per_call = time_calls(prepared, reps)
    head_argmax = time_head_argmax(next(p for p in prepared if p.call.name == "lm_head"), reps)
    weight_copies = {p.call.name: p.copies for p in prepared}
    del graphs, ref, prepared  # free the step's buffers before the other calls
    torch.cuda.empty_cache()
    others = [Prepared(c, dev) for c in other_calls()]
    other = time_calls(others, reps)
    for d in other.values():
        del d["hbm_bytes_counted"]
    del others
    torch.cuda.empty_cache()
    layer = time_decode_layer(dev, 50)
    torch.cuda.empty_cache()
    layer_inside = time_decode_layer(dev, 50, inside=True)
    torch.cuda.empty_cache()
    ceiling = stream_ceiling([d["weight_bytes"] for d in per_call.values()] +
                             [d["weight_bytes"] for d in other.values()], dev)
    torch.cuda.empty_cache()
    for d in list(per_call.values()) + list(other.values()):
        c = ceiling[str(d["weight_bytes"])]
        d["pct_of_stream_ceiling"] = round(c["us"] / d["project_us"] * 100, 1)
    per_rows = rows_summary(per_call, ceiling)

    dom_name = max(per_call, key=lambda n: per_call[n]["project_us"])
    dom = per_call[dom_name]
    achieved = dom["weight_bytes"] / (dom["project_us"] * 1e-6) / 1e9
    traffic = stored_traffic(dom_name)
    dom_ceiling = ceiling[str(dom["weight_bytes"])]
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": f"{dom_name}: rows={dom['rows']} {dom['n']}x{dom['k']} {dom['mode']}",
                "algorithmic_bytes": dom["weight_bytes"],
                "stream_ceiling_GBps": dom_ceiling["GBps"],
                "frac_of_stream_ceiling": round(achieved / dom_ceiling["GBps"], 4)}

    cpu = None if args.no_cpu else cpu_baseline(calls, args.cpu_budget)

    out = {
        "metric": METRIC,
        "value": round(step_bytes / step_s / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": "Q8_0 projection step: decode rows=1 (4096x14336, two-word) + batched decode "
                               "rows=8 (14336x4096 two-word; 4096x14336 two-word + residual) + prefill rows=64 "
                               "(14336x4096, one-word) + LM head on the last row (151936x2048, one-word)",
                   "weight_bytes_per_step": step_bytes, "graph_replay": True,
                   "weight_copies": weight_copies},
        "pct_hbm_peak": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBPS * 100, 1),
        "per_rows": per_rows,
        "per_call": per_call,
        "lm_head_argmax": head_argmax,
        "other_calls": other,
        "stream_ceiling": ceiling,
        "decode_layer": layer,
        "decode_layer_quantize_inside": layer_inside,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
