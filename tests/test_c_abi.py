"""The boundary from C: include/usp.h compiles as strict C99, and a plain C
program linked against libusp.so gets the version and the synchronous
validation errors the header documents (no GPU needed, nothing launched)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
PKG = os.path.join(ROOT, "sequence_ring_attention_amd")
LIB = os.path.join(PKG, "libusp.so")

needs_gcc = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")


@needs_gcc
def test_header_compiles_as_strict_c99():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only", "-x", "c",
                        os.path.join(INC, "usp.h")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@needs_gcc
def test_c_program_calls_the_library(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libusp.so not built")
    exe = str(tmp_path / "abi_check")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", INC,
                        os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", exe, LIB, "-Wl,-rpath," + PKG],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "abi ok"
