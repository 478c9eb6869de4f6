"""Host sanitizer runs, CPU only: AddressSanitizer + UndefinedBehaviorSanitizer.

Two instrumented builds, each run under the CPU tests that exercise it, in a
child process with the matching sanitizer runtime preloaded (leak checking
off: the Python interpreter keeps its allocations to the end by design):
  - the C oracle (gcc -fsanitize=address,undefined) under tests/test_oracle.py;
  - the library's host code (hipcc, -fsanitize= after -Xarch_host, so device
    code is built as usual and never runs here) under tests/test_abi.py,
    which drives every entry point's validation, the size queries, the
    no-op cases and the status strings.
Any sanitizer report ends the child with an error; the test fails with its
output.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _child(env_extra, test_file):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", test_file)]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    text = res.stdout + res.stderr
    assert res.returncode == 0 and "runtime error" not in text and "ERROR: AddressSanitizer" not in text, text[-6000:]
    assert " passed" in text, text[-3000:]


def _gcc_runtime(name):
    return subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build(force=True, sanitize=True, out=str(tmp_path / "libkda_oracle_san.so"))
    _child({"KDA_ORACLE_LIB": lib, "LD_PRELOAD": _gcc_runtime("libasan.so")}, "test_oracle.py")


def test_library_host_code_under_asan_ubsan(tmp_path):
    from chunked_gated_delta_10_amd import build
    rt = build.sanitizer_runtime()
    if not os.path.exists(rt):
        pytest.skip("clang AddressSanitizer runtime not found")
    lib = build.build_sanitized(str(tmp_path / "libkda_san.so"), jobs=min(8, os.cpu_count() or 1))
    _child({"KDA_LIB": lib, "LD_PRELOAD": rt}, "test_abi.py")
