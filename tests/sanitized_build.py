"""Host-code builds with AddressSanitizer and UndefinedBehaviorSanitizer, for
the CPU test that runs the ABI validation, the oracle and the input generator
under them.  CPU only: the GPU library's device code is built as usual, only
its host side (argument validation, dispatch, launchers) is instrumented.
"""
from __future__ import annotations

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# host-only sanitizer flags for hipcc: each -fsanitize= right after -Xarch_host
HIP_HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def clang_asan_runtime() -> str:
    """The ASan runtime of the ROCm clang that hipcc drives (it also carries
    the UBSan handlers)."""
    out = subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        rt = subprocess.run(["/opt/rocm/llvm/bin/clang", "-print-runtime-dir"], capture_output=True, text=True,
                            check=True).stdout.strip()
        out = os.path.join(rt, "libclang_rt.asan-x86_64.so")
    return out


def gcc_runtime(name: str) -> str:
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build_library(out_dir: str) -> str:
    import sys
    sys.path.insert(0, ROOT)
    from q8_projection_amd import build as q8build
    return q8build.build(lib=os.path.join(out_dir, "libq8proj_san.so"), obj_dir=os.path.join(out_dir, "obj"),
                         extra=HIP_HOST_SAN)


def build_oracle_and_synth(out_dir: str) -> dict:
    libs = {}
    for name, src in (("Q8REF_LIB", "oracle/q8ref.c"), ("SYNTH_LIB", "synth/synth.c")):
        out = os.path.join(out_dir, os.path.basename(src).replace(".c", "_san.so"))
        cmd = ["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", *GCC_SAN,
               "-o", out, os.path.join(ROOT, src), "-lm"]
        subprocess.run(cmd, check=True)
        libs[name] = out
    return libs
