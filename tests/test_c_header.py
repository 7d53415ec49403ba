"""The C ABI used from C (CPU only): tests/c/abi_host_check.c is compiled as
strict C99 against include/qlora_nf4.h, linked to the built library and run;
it checks the struct layouts and the host-side entry points."""
import os
import shutil
import subprocess

import pytest

from bit_nf4_quantized_06_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_compiles_as_c99_and_host_calls_work(tmp_path):
    _lib.load()                       # the library is built (raises otherwise)
    libdir = os.path.dirname(_lib.LIB_PATH)
    exe = str(tmp_path / "abi_host_check")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host_check.c"),
                    "-L", libdir, "-l:" + os.path.basename(_lib.LIB_PATH),
                    f"-Wl,-rpath,{libdir}", "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
