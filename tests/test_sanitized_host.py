"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's argument validation and dispatch (its host side; the device code
is built as usual), the CPU oracle and the input generator are rebuilt with
both sanitizers, and their CPU tests run again in a child process against those
builds: any out-of-bounds access, use after free, signed overflow or other
undefined behaviour those tests reach aborts the run.
"""
import os
import subprocess
import sys

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)


def _run(env_extra, preload, tests, timeout):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = " ".join(preload)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *tests]
    proc = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    tail = (proc.stdout + proc.stderr)[-4000:]
    assert proc.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    return tail


def test_abi_validation_under_sanitizers(tmp_path):
    import sanitized_build as sb
    lib = sb.build_library(str(tmp_path))
    out = _run({"Q8PROJ_LIB": lib}, [sb.clang_asan_runtime()], [os.path.join(TESTS, "test_abi_cpu.py")], 600)
    assert " passed" in out


def test_oracle_and_generator_under_sanitizers(tmp_path):
    import sanitized_build as sb
    libs = sb.build_oracle_and_synth(str(tmp_path))
    out = _run(libs, [sb.gcc_runtime("libasan.so"), sb.gcc_runtime("libubsan.so")],
               [os.path.join(TESTS, "test_oracle.py")], 900)
    assert " passed" in out
