"""The C ABI from C: tests/c/abi_consumer.c is compiled with gcc as strict
C99 against include/pdr_splat.h, linked to the built library and run (host
side only, no device)."""
import os
import shutil
import subprocess

import pytest

from differentiable_gaussian_splatting_pdr_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c99_consumer(tmp_path):
    libdir = os.path.dirname(_lib.LIB_PATH)
    exe = str(tmp_path / "abi_consumer")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_consumer.c"),
           "-o", exe, "-L", libdir, "-l:" + os.path.basename(_lib.LIB_PATH),
           "-Wl,-rpath," + libdir, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert "abi consumer ok" in out.stdout
