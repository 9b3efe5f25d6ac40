"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_driver.c calls every entry point of
oracle/nvfp4_oracle.h on inputs whose buffers have exactly the documented
sizes (ragged shapes, row strides above the width, both input types, both
roundings, the Hadamard transform, every layout, zeros of both signs,
subnormals, values near the binary32 maximum).  It is built here with gcc for
the host only, together with the oracle's C source, and any sanitizer report
fails the test.  No GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_sanitize")
    # the sanitizer runtimes are linked statically, so the program needs no
    # particular order of the shared libraries loaded with it
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-static-libasan", "-static-libubsan",
           "-fno-omit-frame-pointer", "-ffp-contract=off", "-Wall", "-Wextra", "-Werror",
           "-o", exe, os.path.join(HERE, "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "nvfp4_oracle.c"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "cannot find -l" in r.stderr and "san" in r.stderr:
        pytest.skip("sanitizer runtime libraries not installed")
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "ok" in run.stdout.split()
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-4000:]
