"""The oracle's C source built with AddressSanitizer and UndefinedBehavior-
Sanitizer, and every oracle pin run against that build in a child process:
an out-of-bounds access, a use after free or undefined behaviour anywhere in
ssm_oracle.c ends the run with a report.  CPU only (gcc, no GPU)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ssm_oracle.c")


def _runtime(gcc, name):
    path = subprocess.run([gcc, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    asan = _runtime(gcc, "libasan.so")
    if asan is None:
        pytest.skip("the AddressSanitizer runtime is not available")
    lib = str(tmp_path / "liboracle_sanitized.so")
    flags = ["-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.run([gcc, *flags, "-o", lib, SRC, "-lm", "-lpthread"], check=True)
    env = dict(os.environ, SSM_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join("tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out
