"""The CPU oracle's pin suite once more, against a build of the oracle
instrumented with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
-fno-sanitize-recover): an out-of-bounds access, a use of freed memory, a
shift past the width of its type or a signed overflow anywhere in the
oracle's bit loops ends the run.  CPU only; the sanitizer runtime is
preloaded into a child interpreter, which is skipped when something else is
already preloaded."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_pin_suite_under_asan_and_ubsan(tmp_path):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("another library is preloaded; not combining it with the sanitizer runtime")
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not found")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan not installed")
    lib = str(tmp_path / "libibp_oracle_sanitized.so")
    subprocess.run([gcc, "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-std=gnu11", "-Wall", "-Wextra", "-shared", "-fPIC",
                    os.path.join(ROOT, "oracle", "ibp_oracle.c"), "-o", lib], check=True)
    env = dict(os.environ, LD_PRELOAD=asan, IBP_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout and "failed" not in r.stdout
