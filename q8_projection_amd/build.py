"""Build libq8proj.so (HIP, gfx950) in-tree with hipcc.

Every translation unit is compiled to an object in parallel (the GEMV and MFMA
kernel templates are instantiated across several units for this), then linked
into one shared library.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libq8proj.so")
# the benchmark's streaming-read ceiling probe, a library of its own
PROBE_LIB = os.path.join(HERE, "libq8probe.so")
PROBE_SOURCES = ["stream_probe.hip"]
SOURCES = ["abi.cpp", "quantize.hip", "gemv.hip", "gemv_f32.hip", "gemv_i8.hip", "gemv_i8x2.hip",
           "gemv_sums.hip", "mma.hip", "mma_sums.hip", "f64mma.hip", "argmax_noalloc.hip"]
ARCH = "gfx950"

# Packed f32 VALU ops are kept out of the device code; the host pass warns that
# it does not know the feature, which is harmless.
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fhip-fp32-correctly-rounded-divide-sqrt", "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str, verbose: bool, obj_dir: str, extra) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *FLAGS, *extra, "-c", "-o", obj, os.path.join(CSRC, src)]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False, jobs: int | None = None, lib: str = LIB, obj_dir: str = OBJ,
          extra=()) -> str:
    """Compile every HIP source for gfx950 into ``lib`` (default ``libq8proj.so``
    in-tree; always recompiles).  ``extra`` flags go to every compile and the
    link (the tests' host-sanitizer build passes host-only flags here)."""
    os.makedirs(obj_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, obj_dir, list(extra)), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("hipcc failed linking libq8proj.so")
    os.replace(tmp, lib)
    if lib == LIB:
        build_probe(verbose)
    return lib


def build_probe(verbose: bool = False) -> str:
    """Compile the benchmark's stream probe into ``libq8probe.so``."""
    objs = [_compile(s, verbose, OBJ, []) for s in PROBE_SOURCES]
    tmp = PROBE_LIB + ".tmp"
    proc = subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                          capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("hipcc failed linking libq8probe.so")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
