"""CPU fp64 oracle of the 2D anisotropic Gaussian splatting layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the library or its binding.
It shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain C, fp64, glibc libm); this module
only builds it with gcc and marshals numpy arrays through ctypes.  What each
function computes, and from which passage of the pages, is stated in the C
file's header:

* ``render``  -- I[b,y,x,c] = sum_n a w, with per-pixel slack (the terms of
  pairs within the truncation-tie band |q - k^2| <= tau k^2) and magnitude
  (sum of |terms|); ``allpairs=True`` evaluates every (pixel, Gaussian) pair
  with no pruning.
* ``grad``    -- the analytic backward dL/d(mu, s, theta, a) with slack and
  magnitude per output.
* ``count_support`` -- per frame, the number of (Gaussian, pixel) pairs
  inside the truncation (the unit of work the benchmark reports).
* ``bin``     -- brute-force (tile, Gaussian) overlap lists, ascending
  Gaussian index, and each Gaussian's pixel box.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liborc.so")
_lib = None

TAU = 1e-4  # relative width of the truncation-tie band |q - k^2| <= TAU k^2


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (fp64, no fast-math, no FMA contraction)."""
    stale = (not os.path.exists(_LIB)
             or os.path.getmtime(_LIB) < os.path.getmtime(_SRC))
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-D_GNU_SOURCE", _SRC, "-o", tmp, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # PDR_ORACLE_LIB: a separately built copy of oracle.c (the sanitizer
        # test loads one built with ASan and UBSan)
        path = os.environ.get("PDR_ORACLE_LIB")
        if not path:
            path = build(force=False)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        lp = ctypes.POINTER(ctypes.c_longlong)
        i, d = ctypes.c_int, ctypes.c_double
        lib.orc_render.argtypes = [dp, i, i, i, i, i, d, d, i, i, dp, dp, dp, lp]
        lib.orc_render.restype = ctypes.c_int
        lib.orc_grad.argtypes = [dp, dp, i, i, i, i, i, d, d, i, dp, dp, dp]
        lib.orc_grad.restype = ctypes.c_int
        lib.orc_bin.argtypes = [dp, i, i, i, i, i, d, i, i, ip, lp, ip, ctypes.c_longlong, ip]
        lib.orc_bin.restype = ctypes.c_longlong
        lib.orc_count_support.argtypes = [dp, i, i, i, i, i, d, i, lp]
        lib.orc_count_support.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a, ct):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ct))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _params64(params):
    p = np.ascontiguousarray(params, dtype=np.float64)
    if p.ndim != 3 or p.shape[2] < 6:
        raise ValueError("params must be [B, N, 5 + C] with C >= 1")
    return p


def render(params, H, W, radius=3.0, tau=TAU, allpairs=False, nthreads=None, extras=True):
    """Return (image, slack, mag, pairs) as fp64 [B,H,W,C] (+ int64 [B]).

    slack holds the |terms| of the pairs in the truncation-tie band."""
    p = _params64(params)
    B, N, P = p.shape
    C = P - 5
    img = np.empty((B, H, W, C), np.float64)
    slk = np.empty_like(img) if extras else None
    mag = np.empty_like(img) if extras else None
    pairs = np.zeros(B, np.int64)
    rc = _load().orc_render(_ptr(p, ctypes.c_double), B, N, H, W, C, float(radius), float(tau),
                            int(bool(allpairs)), int(nthreads or default_threads()),
                            _ptr(img, ctypes.c_double), _ptr(slk, ctypes.c_double),
                            _ptr(mag, ctypes.c_double), _ptr(pairs, ctypes.c_longlong))
    if rc != 0:
        raise ValueError("orc_render failed: %d" % rc)
    return img, slk, mag, pairs


def grad(params, grad_image, H, W, radius=3.0, tau=TAU, nthreads=None, extras=True):
    """Return (grad, slack, mag) as fp64 [B,N,5+C] (slack as in ``render``)."""
    p = _params64(params)
    B, N, P = p.shape
    C = P - 5
    g = np.ascontiguousarray(grad_image, dtype=np.float64)
    if g.shape != (B, H, W, C):
        raise ValueError("grad_image must be [B, H, W, C]")
    out = np.empty_like(p)
    slk = np.empty_like(p) if extras else None
    mag = np.empty_like(p) if extras else None
    rc = _load().orc_grad(_ptr(p, ctypes.c_double), _ptr(g, ctypes.c_double), B, N, H, W, C,
                          float(radius), float(tau), int(nthreads or default_threads()),
                          _ptr(out, ctypes.c_double), _ptr(slk, ctypes.c_double),
                          _ptr(mag, ctypes.c_double))
    if rc != 0:
        raise ValueError("orc_grad failed: %d" % rc)
    return out, slk, mag


def bin(params, H, W, radius=3.0, tile=16, nthreads=None, with_lists=True):
    """Return (counts i32[B, nT], tile_off i64[B*nT+1], list i32[total], rect i32[B,N,4])."""
    p = _params64(params)
    B, N, P = p.shape
    C = P - 5
    nT = ((W + tile - 1) // tile) * ((H + tile - 1) // tile)
    counts = np.zeros((B, nT), np.int32)
    off = np.zeros(B * nT + 1, np.int64)
    rect = np.zeros((B, N, 4), np.int32)
    lib = _load()
    nth = int(nthreads or default_threads())
    tot = lib.orc_bin(_ptr(p, ctypes.c_double), B, N, H, W, C, float(radius), int(tile), nth,
                      _ptr(counts, ctypes.c_int), _ptr(off, ctypes.c_longlong), None, 0,
                      _ptr(rect, ctypes.c_int))
    if tot < 0:
        raise ValueError("orc_bin failed: %d" % tot)
    lst = None
    if with_lists:
        lst = np.zeros(max(int(tot), 1), np.int32)
        tot2 = lib.orc_bin(_ptr(p, ctypes.c_double), B, N, H, W, C, float(radius), int(tile), nth,
                           _ptr(counts, ctypes.c_int), _ptr(off, ctypes.c_longlong),
                           _ptr(lst, ctypes.c_int), lst.size, None)
        if tot2 != tot:
            raise ValueError("orc_bin failed: %d" % tot2)
        lst = lst[:tot]
    return counts, off, lst, rect


def count_support(params, H, W, radius=3.0, nthreads=None):
    """Return int64 [B]: pairs with q <= k^2 per frame."""
    p = _params64(params)
    B, N, P = p.shape
    pairs = np.zeros(B, np.int64)
    rc = _load().orc_count_support(_ptr(p, ctypes.c_double), B, N, H, W, P - 5, float(radius),
                                   int(nthreads or default_threads()),
                                   _ptr(pairs, ctypes.c_longlong))
    if rc != 0:
        raise ValueError("orc_count_support failed: %d" % rc)
    return pairs
