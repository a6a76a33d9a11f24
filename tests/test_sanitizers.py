"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* The library: its sources built by hipcc with the flags of the package's
  build (sanitizers on the host pass only), driven by tests/c/host_sanitize.c
  compiled by ROCm's clang against the same sanitizer runtime.  Every call
  there must be rejected by the host-side checks, so no device is touched.
* The oracle: oracle.c built by gcc with both sanitizers and loaded (through
  PDR_ORACLE_LIB, with the ASan runtime preloaded) by its pin tests and by a
  ragged multi-threaded render / gradient / binning / count pass.

Any out-of-bounds access, use after free or signed overflow on these paths
fails the test.  Skipped where a GPU is visible: the driver's calls are
meant never to reach a device, and this suite is host-only.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}

pytestmark = [
    pytest.mark.slow,
    pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="host-only: run where no GPU is visible"),
]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd[:3]), r.stdout[-4000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not available")
def test_library_host_checks_under_asan_ubsan(tmp_path):
    from differentiable_gaussian_splatting_pdr_amd import build as b
    hipcc = b.hipcc()
    flags = [f for f in b.HIPCC_FLAGS if f != "-shared"]
    san = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([hipcc, *flags, *san, "-I", os.path.join(ROOT, "include"), "-c",
              os.path.join(b.PKG, src), "-o", obj])
        return obj
    with ThreadPoolExecutor(max_workers=min(8, len(b.SOURCES))) as ex:
        objs = list(ex.map(compile_one, b.SOURCES))
    lib = str(tmp_path / "libpdrsplat_san.so")
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib])
    exe = str(tmp_path / "host_sanitize")
    _run([CLANG, "-std=c99", "-g", "-Wall", "-Wextra", "-Werror",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "host_sanitize.c"),
          "-o", exe, lib, "-Wl,-rpath," + str(tmp_path), "-lm"])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env={**os.environ, **SAN_ENV})
    assert r.returncode == 0, r.stdout + r.stderr[-6000:]
    assert "host sanitize ok" in r.stdout
    assert "runtime error" not in r.stderr


_RAGGED = r"""
import numpy as np, oracle
from differentiable_gaussian_splatting_pdr_amd import workloads
assert oracle._load()._name == %r
for seed, (B, N, H, W, C) in enumerate([(2, 37, 23, 41, 3), (1, 5, 1, 1, 1), (3, 64, 17, 50, 2)]):
    p, g = workloads.make_custom(B, N, H, W, C, seed=seed, s_range=(0.3, 9.0), mean_margin=6.0)
    for threads in (1, 3):
        img, slk, mag, pairs = oracle.render(p, H, W, 3.0, nthreads=threads)
        ref, _, _, _ = oracle.render(p, H, W, 3.0, allpairs=True, nthreads=threads)
        assert np.allclose(img, ref, rtol=0, atol=1e-12)
        oracle.grad(p, g, H, W, 3.0, nthreads=threads)
        oracle.bin(p, H, W, 3.0, tile=16, nthreads=threads)
        oracle.count_support(p, H, W, 3.0, nthreads=threads)
print("oracle ragged ok")
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "liborc_san.so")
    _run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-D_GNU_SOURCE", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm", "-lpthread"])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    env = {**os.environ, **SAN_ENV, "LD_PRELOAD": asan, "PDR_ORACLE_LIB": lib,
           "PYTHONPATH": ROOT}
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr
    r = subprocess.run([sys.executable, "-c", _RAGGED % lib], capture_output=True, text=True,
                       timeout=600, env=env, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "oracle ragged ok" in r.stdout and "runtime error" not in r.stderr
