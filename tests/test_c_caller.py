"""The C ABI from plain C: tests/c/abi_from_c.c includes only include/fp8mi.h
(compiled as strict C99 with warnings as errors, so the header is valid C) and
links only the built library; it checks the version, the status strings and
host-side argument refusals, none of which needs a GPU."""

import os
import shutil
import subprocess

import pytest

import fp8_precision_numerics_amd as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_plain_c_caller(tmp_path):
    lib = fm.load_library()
    libdir = os.path.dirname(lib._name)
    exe = tmp_path / "abi_from_c"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L", libdir, "-lfp8mi", f"-Wl,-rpath,{libdir}",
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "UNEXPECTED" not in run.stdout
