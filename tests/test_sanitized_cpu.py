"""The C-ABI tests that need no GPU, run against a build of the library whose
host code is compiled with AddressSanitizer and UndefinedBehaviorSanitizer
(argument validation, the fp64 weight preparation, error paths): any
out-of-bounds access, use after free or undefined behaviour in them stops the
run with a report."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    return shutil.which("hipcc") or (os.path.exists("/opt/rocm/bin/hipcc") and "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not _hipcc(), reason="no ROCm toolchain to build the sanitized library")
def test_abi_tests_under_asan_and_ubsan(tmp_path):
    from flow_matching_action_amd import build as b
    lib = b.build(sanitize=True, out=str(tmp_path / "libpi_ae_san.so"))
    env = dict(os.environ)
    env.update({"PI_AE_LIB": lib, "LD_PRELOAD": b.sanitizer_runtime(),
                # the interpreter itself is not instrumented: its own allocations are not leak-checked
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
