"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: the pin
suite (tests/test_oracle_pins.py) runs in a child process against an oracle
library built with -fsanitize=address,undefined (-fno-sanitize-recover), with
libasan preloaded.  Any out-of-bounds access, use after free or undefined
behaviour in oracle.c aborts the child.  CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the sanitizer oracle")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _libasan()
    if asan is None:
        pytest.skip("libasan is not installed with gcc")
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x", "-q",
           "-p", "no:cacheprovider", "-m", "not gpu"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
