"""ctypes binding of ``libpdrsplat.so`` (the C ABI in ``include/pdr_splat.h``).

Argument marshalling only: every function here forwards to the entry point of
the same name and turns a negative status into :class:`PdrError`.  Pointers
are passed as integers (device addresses, ``hipStream_t`` handles).  There is
no fallback: if the library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpdrsplat.so")

PDR_OK = 0
PDR_ERR_INVALID_ARG = -1
PDR_ERR_WORKSPACE = -2
PDR_ERR_HIP = -3
PDR_ERR_OVERFLOW = -4
PDR_ERR_STALE = -5

EXPORTED = (
    "pdr_splat_tile_size",
    "pdr_splat_bin_variant",
    "pdr_splat_backward_splits",
    "pdr_splat_count_support",
    "pdr_splat_workspace_bytes",
    "pdr_splat_forward",
    "pdr_splat_forward_noalloc",
    "pdr_splat_noalloc_scratch_bytes",
    "pdr_splat_backward",
    "pdr_splat_bin",
    "pdr_splat_check",
    "pdr_splat_status_async",
    "pdr_splat_status_string",
    "pdr_splat_timing",
    "pdr_splat_timing_read",
    "pdr_splat_kernel_name",
    "pdr_loss_workspace_bytes",
    "pdr_loss_l1_ssim",
    "pdr_splat_forward_concat",
    "pdr_splat_backward_concat",
    "pdr_grid_init",
    "pdr_params_activate",
    "pdr_params_activate_backward",
    "pdr_splat_forward_fmt",
    "pdr_splat_backward_fmt",
    "pdr_splat_backward_algo",
)

KERNEL_COUNT = 14


class PdrError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (%d)" % (where, status_string(status), status))


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        # One HIP runtime per process: PyTorch's ROCm wheel bundles its own
        # libamdhip64 (loaded under a different file name), so if this library
        # came first it would bind the system runtime and torch would load a
        # second one beside it -- torch's streams and allocations would then
        # be foreign handles to this library's launches.  With torch loaded
        # first, this library's libamdhip64.so.7 resolves to torch's copy.
        try:
            import torch  # noqa: F401
        except ImportError:   # a torch-free host (C ABI checks only)
            pass
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libpdrsplat.so is not built (expected at %s); run "
                "`python -m differentiable_gaussian_splatting_pdr_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        i, ll, f, vp, sz = ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
        L.pdr_splat_tile_size.argtypes = []
        L.pdr_splat_tile_size.restype = i
        L.pdr_splat_bin_variant.argtypes = [i, i, i, i]
        L.pdr_splat_bin_variant.restype = i
        L.pdr_splat_backward_splits.argtypes = [i, i, i, i]
        L.pdr_splat_backward_splits.restype = i
        L.pdr_splat_count_support.argtypes = [vp, i, i, i, i, i, f, vp, vp, sz, vp]
        L.pdr_splat_count_support.restype = i
        L.pdr_splat_workspace_bytes.argtypes = [i, i, i, i, i, ll]
        L.pdr_splat_workspace_bytes.restype = ll
        L.pdr_splat_forward.argtypes = [vp, vp, i, i, i, i, i, f, vp, sz, vp]
        L.pdr_splat_forward.restype = i
        L.pdr_splat_forward_noalloc.argtypes = [vp, vp, i, i, i, i, i, f, vp, vp]
        L.pdr_splat_forward_noalloc.restype = i
        L.pdr_splat_noalloc_scratch_bytes.argtypes = []
        L.pdr_splat_noalloc_scratch_bytes.restype = ll
        L.pdr_splat_backward.argtypes = [vp, vp, vp, i, i, i, i, i, f, vp, sz, i, vp]
        L.pdr_splat_backward.restype = i
        L.pdr_splat_bin.argtypes = [vp, i, i, i, i, i, f, vp, vp, ll, vp, sz, vp]
        L.pdr_splat_bin.restype = i
        L.pdr_splat_check.argtypes = [vp, vp, ctypes.POINTER(ll)]
        L.pdr_splat_check.restype = i
        L.pdr_splat_status_async.argtypes = [vp, vp, vp]
        L.pdr_splat_status_async.restype = i
        L.pdr_splat_status_string.argtypes = [i]
        L.pdr_splat_status_string.restype = ctypes.c_char_p
        L.pdr_splat_timing.argtypes = [i]
        L.pdr_splat_timing.restype = i
        L.pdr_splat_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ll), i]
        L.pdr_splat_timing_read.restype = i
        L.pdr_splat_kernel_name.argtypes = [i]
        L.pdr_splat_kernel_name.restype = ctypes.c_char_p
        L.pdr_loss_workspace_bytes.argtypes = [i, i, i, i]
        L.pdr_loss_workspace_bytes.restype = ll
        L.pdr_loss_l1_ssim.argtypes = [vp, vp, i, i, i, i, f, f, f, vp, vp, vp, sz, vp]
        L.pdr_loss_l1_ssim.restype = i
        L.pdr_splat_forward_concat.argtypes = [vp, vp, i, vp, i, i, i, i, i, f, vp, sz, vp]
        L.pdr_splat_forward_concat.restype = i
        L.pdr_splat_backward_concat.argtypes = [vp, vp, i, vp, vp, i, i, i, i, i, f, vp, sz, i,
                                                vp]
        L.pdr_splat_backward_concat.restype = i
        L.pdr_grid_init.argtypes = [vp, i, i, i, i, i, i, f, vp, vp]
        L.pdr_grid_init.restype = i
        L.pdr_params_activate.argtypes = [vp, vp, i, i, i, i, i, i, vp]
        L.pdr_params_activate.restype = i
        L.pdr_params_activate_backward.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp]
        L.pdr_params_activate_backward.restype = i
        L.pdr_splat_forward_fmt.argtypes = [vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
        L.pdr_splat_forward_fmt.restype = i
        L.pdr_splat_backward_fmt.argtypes = [vp, vp, i, vp, i, i, i, i, i, f, vp, sz, i, vp]
        L.pdr_splat_backward_fmt.restype = i
        L.pdr_splat_backward_algo.argtypes = [vp, vp, i, vp, i, i, i, i, i, f, vp, sz, i, i, vp]
        L.pdr_splat_backward_algo.restype = i
        _lib = L
    return _lib


def _raise(rc: int, where: str) -> int:
    if rc < 0:
        raise PdrError(rc, where)
    return rc


def status_string(status: int) -> str:
    return lib().pdr_splat_status_string(int(status)).decode()


def pdr_splat_tile_size() -> int:
    return lib().pdr_splat_tile_size()


PDR_BIN_MEMBERS, PDR_BIN_COLUMNS, PDR_BIN_TWO_LEVEL = 1, 2, 4


def pdr_splat_count_support(params, B, N, H, W, C, radius, count, workspace, workspace_bytes,
                            stream=None) -> int:
    return _raise(lib().pdr_splat_count_support(params, B, N, H, W, C, float(radius), count,
                                                workspace, workspace_bytes, stream),
                  "pdr_splat_count_support")


def pdr_splat_bin_variant(B, N, H, W) -> int:
    """Bit set of PDR_BIN_* for the binning a problem of this size takes."""
    return _raise(lib().pdr_splat_bin_variant(B, N, H, W), "pdr_splat_bin_variant")


def pdr_splat_backward_splits(B, N, H, W) -> int:
    return _raise(lib().pdr_splat_backward_splits(B, N, H, W), "pdr_splat_backward_splits")


def pdr_splat_workspace_bytes(B, N, H, W, C, max_pairs) -> int:
    return _raise(lib().pdr_splat_workspace_bytes(B, N, H, W, C, int(max_pairs)),
                  "pdr_splat_workspace_bytes")


def pdr_splat_forward(params, image, B, N, H, W, C, radius, workspace, workspace_bytes, stream):
    return _raise(lib().pdr_splat_forward(params, image, B, N, H, W, C, float(radius), workspace,
                                          workspace_bytes, stream), "pdr_splat_forward")


def pdr_splat_forward_noalloc(params, image, B, N, H, W, C, radius, status, stream):
    """Forward with the library's static per-GPU scratch (no workspace, no
    allocation); status: device pointer to one int (PDR_OK / PDR_ERR_OVERFLOW)."""
    return _raise(lib().pdr_splat_forward_noalloc(params, image, B, N, H, W, C, float(radius),
                                                  status, stream), "pdr_splat_forward_noalloc")


def pdr_splat_noalloc_scratch_bytes() -> int:
    return int(lib().pdr_splat_noalloc_scratch_bytes())


def pdr_splat_backward(params, grad_image, grad_params, B, N, H, W, C, radius, workspace,
                       workspace_bytes, reuse_binning, stream):
    return _raise(lib().pdr_splat_backward(params, grad_image, grad_params, B, N, H, W, C,
                                           float(radius), workspace, workspace_bytes,
                                           int(reuse_binning), stream), "pdr_splat_backward")


def pdr_splat_bin(params, B, N, H, W, C, radius, tile_off, tile_list, cap, workspace,
                  workspace_bytes, stream):
    return _raise(lib().pdr_splat_bin(params, B, N, H, W, C, float(radius), tile_off, tile_list,
                                      int(cap), workspace, workspace_bytes, stream),
                  "pdr_splat_bin")


def pdr_splat_check(workspace, stream):
    """Return (status, pairs_needed); the status is not raised."""
    n = ctypes.c_longlong(0)
    rc = lib().pdr_splat_check(workspace, stream, ctypes.byref(n))
    return rc, n.value


def pdr_splat_status_async(workspace, out, stream):
    """Enqueue the status report of the last call into out (two int64)."""
    return _raise(lib().pdr_splat_status_async(workspace, out, stream), "pdr_splat_status_async")


def pdr_splat_timing(enable: bool) -> bool:
    return bool(lib().pdr_splat_timing(int(bool(enable))))


def pdr_splat_kernel_name(kid: int) -> str:
    return lib().pdr_splat_kernel_name(int(kid)).decode()


def pdr_splat_timing_read(reset: bool = True):
    """Return {kernel name: (total_ms, launches)} accumulated since the last reset."""
    ms = (ctypes.c_double * KERNEL_COUNT)()
    cnt = (ctypes.c_longlong * KERNEL_COUNT)()
    _raise(lib().pdr_splat_timing_read(ms, cnt, int(bool(reset))), "pdr_splat_timing_read")
    return {pdr_splat_kernel_name(k): (ms[k], cnt[k]) for k in range(KERNEL_COUNT)}


def pdr_loss_workspace_bytes(B, H, W, C) -> int:
    return _raise(lib().pdr_loss_workspace_bytes(B, H, W, C), "pdr_loss_workspace_bytes")


def pdr_loss_l1_ssim(image, target, B, H, W, C, lam, c1, c2, grad_image, loss, workspace,
                     workspace_bytes, stream):
    return _raise(lib().pdr_loss_l1_ssim(image, target, B, H, W, C, float(lam), float(c1),
                                         float(c2), grad_image, loss, workspace, workspace_bytes,
                                         stream), "pdr_loss_l1_ssim")


def pdr_splat_forward_concat(params, pixel, Cp, out, B, N, H, W, C, radius, workspace,
                             workspace_bytes, stream):
    return _raise(lib().pdr_splat_forward_concat(params, pixel, Cp, out, B, N, H, W, C,
                                                 float(radius), workspace, workspace_bytes,
                                                 stream), "pdr_splat_forward_concat")


def pdr_splat_backward_concat(params, grad_out, Cp, grad_params, grad_pixel, B, N, H, W, C,
                              radius, workspace, workspace_bytes, reuse_binning, stream):
    return _raise(lib().pdr_splat_backward_concat(params, grad_out, Cp, grad_params, grad_pixel,
                                                  B, N, H, W, C, float(radius), workspace,
                                                  workspace_bytes, int(reuse_binning), stream),
                  "pdr_splat_backward_concat")


def pdr_grid_init(raw, B, gx, gy, H, W, C, init_scale, image, stream):
    return _raise(lib().pdr_grid_init(raw, B, gx, gy, H, W, C, float(init_scale), image, stream),
                  "pdr_grid_init")


def pdr_params_activate(raw, params, B, gx, gy, H, W, C, stream):
    return _raise(lib().pdr_params_activate(raw, params, B, gx, gy, H, W, C, stream),
                  "pdr_params_activate")


def pdr_params_activate_backward(raw, grad_params, grad_raw, B, gx, gy, H, W, C, stream):
    return _raise(lib().pdr_params_activate_backward(raw, grad_params, grad_raw, B, gx, gy, H, W,
                                                     C, stream),
                  "pdr_params_activate_backward")


PDR_FMT_F32, PDR_FMT_F16, PDR_FMT_BF16 = 0, 1, 2


def pdr_splat_forward_fmt(params, image, image_format, B, N, H, W, C, radius, workspace,
                          workspace_bytes, stream):
    return _raise(lib().pdr_splat_forward_fmt(params, image, int(image_format), B, N, H, W, C,
                                              float(radius), workspace, workspace_bytes, stream),
                  "pdr_splat_forward_fmt")


def pdr_splat_backward_fmt(params, grad_image, grad_format, grad_params, B, N, H, W, C, radius,
                           workspace, workspace_bytes, reuse_binning, stream):
    return _raise(lib().pdr_splat_backward_fmt(params, grad_image, int(grad_format), grad_params,
                                               B, N, H, W, C, float(radius), workspace,
                                               workspace_bytes, int(reuse_binning), stream),
                  "pdr_splat_backward_fmt")


PDR_BWD_AUTO, PDR_BWD_TILE, PDR_BWD_SPAN = 0, 1, 2


def pdr_splat_backward_algo(params, grad_image, grad_format, grad_params, B, N, H, W, C, radius,
                            workspace, workspace_bytes, reuse_binning, algo, stream):
    return _raise(lib().pdr_splat_backward_algo(params, grad_image, int(grad_format), grad_params,
                                                B, N, H, W, C, float(radius), workspace,
                                                workspace_bytes, int(reuse_binning), int(algo),
                                                stream), "pdr_splat_backward_algo")
