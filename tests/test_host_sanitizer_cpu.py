"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the host-sanitized variant of the library (every -fsanitize applies
to the host pass only; the device code is the same) and runs the CPU-only
ABI and binding tests against it in a child process with the ASan runtime
preloaded. Those tests drive the validation, workspace-size and error paths
of every entry point with host memory, so an out-of-bounds access, a use
after free or undefined behaviour (overflow, bad shift, misaligned access)
in that code aborts the child with a report. No GPU is needed.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="no hipcc")
def test_abi_host_code_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from learnable_polynomial_feature_amd import build as B

    lib = B.build(host_sanitize=True)
    asan = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True, check=True).stdout.strip()
    assert os.path.exists(asan), asan
    env = dict(os.environ, LD_PRELOAD=asan, LLOPS_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p",
                        "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                        os.path.join(ROOT, "tests", "test_binding_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail  # UBSan's report line
