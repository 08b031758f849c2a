"""The CPU oracle under the sanitizers (host code only; no GPU involved).

UndefinedBehaviorSanitizer: the oracle library is rebuilt with
-fsanitize=undefined (any finding aborts) and the whole pin suite runs
against that copy in a subprocess.  AddressSanitizer: the oracle is compiled
together with tests/sanitize_driver.c into one executable, which calls every
oracle function on small, empty and malformed shapes; ASan reports any
out-of-bounds access or leak and makes the run fail.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
UBSAN = ["-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def test_pins_pass_under_ubsan(tmp_path):
    lib = oracle.build(oracle.SOURCE, str(tmp_path / "liboracle_ubsan.so"), extra_flags=UBSAN)
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="4",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_driver_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_driver")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off",
           "-fsanitize=address", *UBSAN, "-o", exe, oracle.SOURCE,
           os.path.join(ROOT, "tests", "sanitize_driver.c"), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "sanitize driver ok" in r.stdout
