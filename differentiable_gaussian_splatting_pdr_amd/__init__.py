"""MI355X (gfx950) differentiable 2D anisotropic Gaussian splatting.

The forward renders per-frame sets of Gaussians (mean, per-axis scale,
rotation, C channel amplitudes) onto an H x W x C grid by additive
accumulation of truncated Gaussian kernels; the backward returns gradients
for every parameter.  The computation runs in hand-written HIP kernels for
gfx950 behind the C ABI of ``include/pdr_splat.h``; this package is the
Python binding (``_lib``: ctypes, same names as the C entry points;
``splat``: PyTorch tensors, workspace handling, autograd).
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    PdrError,
    pdr_splat_backward,
    pdr_splat_bin,
    pdr_splat_bin_variant,
    pdr_splat_check,
    pdr_splat_forward,
    pdr_splat_tile_size,
    pdr_splat_workspace_bytes,
    status_string,
)

__all__ = [
    "LIB_PATH", "PdrError", "pdr_splat_backward", "pdr_splat_bin", "pdr_splat_bin_variant",
    "pdr_splat_check",
    "pdr_splat_forward", "pdr_splat_tile_size", "pdr_splat_workspace_bytes", "status_string",
]
