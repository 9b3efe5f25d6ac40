"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer.

The ABI layer (csrc/nvfp4_api.hip) is compiled with both sanitizers on its
host code only (each -fsanitize option placed after -Xarch_host, so no
device code is instrumented) and linked with the library's kernel objects
from its regular build; tests/abi_sanitize_driver.c, a C program, is built
against it with the same sanitizers and calls every entry point with
arguments that validation must refuse, checking each status.  Nothing is
launched.  Any wrong status or sanitizer report fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

from bit_block_scaled_quantize_amd import build as B  # noqa: E402

SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def test_abi_validation_under_address_and_ub_sanitizers(tmp_path):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or "/opt/rocm/lib/llvm/bin/clang"
    others = [os.path.join(B.BUILD, s.replace(".hip", ".o")) for s in B.SOURCES if s != "nvfp4_api.hip"]
    if not all(os.path.exists(o) for o in others):
        pytest.skip("the library's kernel objects are not built (run __graft_entry__.build())")
    obj = str(tmp_path / "nvfp4_api_san.o")
    r = subprocess.run([hipcc] + B.flags() + SAN_HOST + ["-c", os.path.join(B.CSRC, "nvfp4_api.hip"), "-o", obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = str(tmp_path / "libnvfp4_san.so")
    r = subprocess.run([hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", lib, obj] + others,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_sanitize")
    r = subprocess.run([clang, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror", "-I", B.INCLUDE, "-o", exe,
                        os.path.join(HERE, "abi_sanitize_driver.c"), "-L", str(tmp_path), "-lnvfp4_san",
                        "-Wl,-rpath," + str(tmp_path)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # leak checking is off: the HIP runtime the library links keeps allocations
    # of its own until exit
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "ok" in run.stdout.split()
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-4000:]
