"""The host side of the C ABI under the address and undefined-behaviour
sanitizers: the library is rebuilt with its host code instrumented (device
code unchanged), and the CPU tests that call into it (argument checks, size
queries, the host page table of the residency manager) run again in a child
process with the sanitizer runtime preloaded.  Any heap overflow,
use-after-free or undefined behaviour in the host code aborts that process."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_under_asan_and_ubsan():
    from lora_adapter_amd import build
    rt = build.asan_runtime()
    if not rt:
        pytest.skip("no clang address sanitizer runtime in this toolchain")
    lib = build.build_sanitized()
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "LORA_ADAPTER_LIB": lib,
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi_cpu.py"),
           os.path.join(ROOT, "tests", "test_residency_oracle.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
