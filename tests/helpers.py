"""Shared test helpers: run the HIP path through the C ABI on numpy inputs and
compare it with the oracle at the stated tolerance.

Tolerance (the pages fix none for the renderer; 1e-4 relative / 1e-5
absolute is the target stated for the fp32 outputs), elementwise, with ref
the fp64 oracle:

  image:  |gpu - ref| <= 1e-5 + 1e-4 |ref| + slack
  grads:  |gpu - ref| <= 1e-5 + 1e-4 max(|ref|, 1e-2 mag) + slack

slack is the summed |term| of the (Gaussian, pixel) pairs within 1e-4 k^2 of
the truncation edge, where either side is a correct result; mag is the
summed |term| of the output.  A gradient is a signed sum of up to thousands
of terms: where it cancels to below 1e-2 of its magnitude, 1e-4 of |ref|
would ask for more than single-precision terms can give, and the bound
falls back to 1e-6 of the magnitude (1e-4 of 1e-2 mag).  check_grad counts
and prints those outputs.
"""
from __future__ import annotations

import numpy as np

ATOL = 1e-5
RTOL = 1e-4
CANCEL = 1e-2   # a gradient below this fraction of its magnitude counts as cancelling


def gpu_forward_backward(params, grad_image, H, W, radius=3.0, reuse=True, algo="tile"):
    """Run forward then backward through the library; numpy in, numpy out.
    algo: "tile" (the tile raster, whatever the library default would pick
    for the size), None (the library default) or a PDR_BWD_* value."""
    import torch
    from differentiable_gaussian_splatting_pdr_amd import _lib, splat

    if algo == "tile":
        algo = _lib.PDR_BWD_TILE

    dev = torch.device("cuda:0")
    p = torch.from_numpy(np.ascontiguousarray(params, dtype=np.float32)).to(dev)
    image, ws = splat.forward(p, H, W, radius)
    out = {"image": image.cpu().numpy()}
    if grad_image is not None:
        g = torch.from_numpy(np.ascontiguousarray(grad_image, dtype=np.float32)).to(dev)
        gp = splat.backward(p, g, H, W, radius, workspace=ws, reuse_binning=reuse, algo=algo)
        out["grad"] = gp.cpu().numpy()
    torch.cuda.synchronize()
    return out


def gpu_bin(params, H, W, radius=3.0):
    import torch
    from differentiable_gaussian_splatting_pdr_amd import splat

    p = torch.from_numpy(np.ascontiguousarray(params, dtype=np.float32)).to("cuda:0")
    off, lst = splat.bin_lists(p, H, W, radius)
    return off.cpu().numpy().astype(np.int64), lst.cpu().numpy()


def check_close(gpu, ref, scale, slack, what, rtol=RTOL, atol=ATOL):
    gpu = np.asarray(gpu, np.float64)
    err = np.abs(gpu - ref)
    bound = atol + rtol * scale + slack
    bad = ~(err <= bound)  # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[:5]
        rows = ["%s gpu=%r ref=%r scale=%r slack=%r" % (tuple(i), gpu[tuple(i)], ref[tuple(i)],
                                                         scale[tuple(i)], slack[tuple(i)])
                for i in idx]
        raise AssertionError("%s: %d of %d outside tolerance; max err %.3g\n  %s" % (
            what, int(bad.sum()), bad.size, float(np.nanmax(err)), "\n  ".join(rows)))
    return float(np.max(err / (atol + rtol * scale + slack))) if err.size else 0.0


def check_grad(gpu, ref, mag, slack, what, rtol=RTOL, atol=ATOL, verbose=True):
    """Gradients: 1e-4 of max(|ref|, 1e-2 mag) + 1e-5 + slack (module doc).
    Returns (worst err/bound ratio, number of outputs on the cancelling
    fallback)."""
    scale = np.maximum(np.abs(ref), CANCEL * mag)
    ratio = check_close(gpu, ref, scale, slack, what, rtol=rtol, atol=atol)
    n_canc = int((np.abs(ref) < CANCEL * mag).sum())
    if verbose:
        print("%s: %d of %d outputs cancel below %g of their magnitude; worst ratio %.3g" % (
            what, n_canc, np.size(ref), CANCEL, ratio))
    return ratio, n_canc


def check_against_oracle(orc, params, grad_image, H, W, radius=3.0, frames=None, gpu=None):
    """Compare image and gradients (optionally on a subset of frames)."""
    if gpu is None:
        gpu = gpu_forward_backward(params, grad_image, H, W, radius)
    sel = slice(None) if frames is None else frames
    p = params[sel]
    img, slk, mag, pairs = orc.render(p, H, W, radius)
    r_img = check_close(gpu["image"][sel], img, np.abs(img), slk, "image")
    out = {"image_ratio": r_img, "pairs": int(pairs.sum())}
    if grad_image is not None:
        gr, gsl, gmag = orc.grad(p, grad_image[sel], H, W, radius)
        out["grad_ratio"], out["grad_cancelling"] = check_grad(gpu["grad"][sel], gr, gmag, gsl, "grad")
    return out


def make_needles(seed=33, B=2, N=150, H=72, W=88, C=3):
    """Long thin rotated Gaussians (anisotropy ~13:1 to 800:1) with means on
    and near 8-pixel unit corners, every seventh on an exact diagonal: the
    thin axis's whitened coordinate cancels to near zero over the support,
    the hardest case for single-precision whitening."""
    from differentiable_gaussian_splatting_pdr_amd import workloads
    rng = np.random.default_rng(seed)
    p, g = workloads.make_custom(B, N, H, W, C, seed=seed)
    p[:, :, 0] = rng.integers(0, W // 8 + 1, (B, N)) * 8 + rng.choice([0.0, 0.5, 1e-3, -0.3], (B, N))
    p[:, :, 1] = rng.integers(0, H // 8 + 1, (B, N)) * 8 + rng.choice([0.0, 0.5, -1e-3, 0.3], (B, N))
    p[:, :, 2] = rng.uniform(8.0, 40.0, (B, N))
    p[:, :, 3] = np.exp(rng.uniform(np.log(0.05), np.log(0.6), (B, N)))
    p[:, :, 4] = rng.uniform(0.0, np.pi, (B, N))
    p[:, ::7, 4] = np.pi / 4
    return p.astype(np.float32), g.astype(np.float32), H, W


def tile_size():
    from differentiable_gaussian_splatting_pdr_amd import _lib
    return _lib.pdr_splat_tile_size()


def check_lists(orc, params, H, W, radius=3.0, gpu=None):
    off_g, lst_g = gpu if gpu is not None else gpu_bin(params, H, W, radius)
    counts, off, lst, _ = orc.bin(params, H, W, radius, tile=tile_size())
    assert np.array_equal(off_g, off), "tile offsets differ"
    assert np.array_equal(lst_g, lst), "tile lists differ"
    return int(off[-1])


def quantize(x, fmt):
    """Round float32 values to the storage format (round to nearest even) and
    return them as float32; fmt 'f16' or 'bf16'."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if fmt == "f16":
        return x.astype(np.float16).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16          # bfloat16: keep the top 16 bits, RNE
    return (u.astype(np.uint32) << 16).view(np.float32)


def format_spacing(ref, fmt):
    """Distance between adjacent values of the format around |ref| (float64)."""
    a = np.abs(np.asarray(ref, np.float64))
    if fmt == "f16":
        return np.spacing(a.astype(np.float16)).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)
