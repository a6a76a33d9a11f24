"""The C ABI from C: tests/c/abi_consumer.c is compiled with gcc as strict
C99 against include/pdr_splat.h, linked to the built library and run (host
side only, no device); tests/c/gpu_consumer.c renders through the ABI on
the GPU from plain C (HIP runtime for memory and a stream, no torch) and
its image and gradients are checked against the oracle."""
import os
import shutil
import subprocess

import numpy as np

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


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_program_renders_on_the_gpu(tmp_path, orc):
    from differentiable_gaussian_splatting_pdr_amd import workloads
    from helpers import check_grad, check_close
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    libdir = os.path.dirname(_lib.LIB_PATH)
    exe = str(tmp_path / "gpu_consumer")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "gpu_consumer.c"), "-o", exe,
           "-L", libdir, "-l:" + os.path.basename(_lib.LIB_PATH), "-Wl,-rpath," + libdir,
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    B, N, H, W, C, radius = 3, 400, 45, 70, 3, 3.0
    p, g = workloads.make_custom(B, N, H, W, C, seed=31, s_range=(0.4, 7.0), mean_margin=4.0)
    src, dst = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    with open(src, "wb") as fh:
        np.array([B, N, H, W, C], np.int32).tofile(fh)
        np.array([radius], np.float32).tofile(fh)
        np.ascontiguousarray(p, np.float32).tofile(fh)
        np.ascontiguousarray(g, np.float32).tofile(fh)
    out = subprocess.run([exe, src, dst], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert "gpu consumer ok (2 attempts" in out.stdout, out.stdout   # one overflow, one regrow
    raw = np.fromfile(dst, np.uint8)
    ni, nparam = B * H * W * C, B * N * (5 + C)
    image = raw[:ni * 4].view(np.float32).reshape(B, H, W, C)
    grad = raw[ni * 4:(ni + nparam) * 4].view(np.float32).reshape(B, N, 5 + C)
    pairs = int(raw[(ni + nparam) * 4:].view(np.int64)[0])
    _, off, _, _ = orc.bin(p, H, W, tile=_lib.pdr_splat_tile_size())
    assert pairs == off[-1]
    ref, slk, _, _ = orc.render(p, H, W, radius)
    check_close(image, ref, np.abs(ref), slk, "image from C")
    gr, gsl, gmag = orc.grad(p, g, H, W, radius)
    check_grad(grad, gr, gmag, gsl, "grad from C")
