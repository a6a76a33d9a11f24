"""Tolerance study of reduced-precision image storage (run on a GPU host):

    python tests/precision_study.py > study.md

For the 384-frame 128x128x3 benchmark batch it renders with the image stored
as fp32, fp16 and bf16, and runs the backward with dL/dI stored the same
way, then reports on sampled frames against the fp64 oracle: the image
error (max, and in spacings of the format), and how far the gradients move
when dL/dI is rounded to the format (relative to the gradients' magnitude,
the sum of |terms|).  It also times the rasters per format (20 steps, HIP
events around every launch).  Test infrastructure: it imports the oracle.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
from differentiable_gaussian_splatting_pdr_amd import _lib, splat, workloads  # noqa: E402
from helpers import format_spacing, quantize  # noqa: E402

FRAMES = [0, 95, 191, 287, 383]


def main():
    oracle.build(force=False)
    wl, params, G = workloads.make_inputs(2)
    H, W = wl.H, wl.W
    dev = torch.device("cuda:0")
    p = torch.from_numpy(params).to(dev)
    ref, slk, _, _ = oracle.render(params[FRAMES], H, W, 3.0)
    g_exact, _, gmag = oracle.grad(params[FRAMES], G[FRAMES], H, W, 3.0)
    rows, times = [], []
    for name, dt, fmt in (("fp32", torch.float32, None), ("fp16", torch.float16, "f16"),
                          ("bf16", torch.bfloat16, "bf16")):
        Gq = G if fmt is None else quantize(G, fmt)
        gt = torch.from_numpy(Gq).to(dev).to(dt)
        img, ws = splat.forward(p, H, W, dtype=dt)
        gp = splat.backward(p, gt, H, W, workspace=ws, reuse_binning=True)
        im = img.float().cpu().numpy()[FRAMES].astype(np.float64)
        err = np.abs(im - ref)
        sp = format_spacing(ref, fmt) if fmt else np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        big = np.abs(ref) >= 0.01   # away from zero, where fp32 error dominates any spacing
        gdev = np.abs(gp.cpu().numpy()[FRAMES] - g_exact) / np.maximum(gmag, 1e-30)
        rows.append("| %s | %.3g | %.3g | %.2f | %.3g | %.3g |" % (
            name, err.max(), (err / np.maximum(np.abs(ref), 1e-3)).max(), (err / sp)[big].max(),
            np.median(gdev), gdev.max()))
        # timing
        for _ in range(3):
            splat.forward(p, H, W, workspace=ws, image=img)
            splat.backward(p, gt, H, W, workspace=ws, reuse_binning=True, check=False)
        torch.cuda.synchronize()
        _lib.pdr_splat_timing(True)
        _lib.pdr_splat_timing_read(reset=True)
        for _ in range(20):
            splat.forward(p, H, W, workspace=ws, image=img)
            splat.backward(p, gt, H, W, workspace=ws, reuse_binning=True, check=False)
        torch.cuda.synchronize()
        t = _lib.pdr_splat_timing_read(reset=True)
        _lib.pdr_splat_timing(False)
        avg = lambda k: t[k][0] / t[k][1] * 1e3
        times.append("| %s | %d | %.1f | %.1f |" % (name, {"fp32": 4, "fp16": 2, "bf16": 2}[name] * im.size // len(FRAMES) * wl.B // 10**6,
                                                   avg("forward_raster"), avg("backward_raster")))
    print("# Reduced-precision image storage, 384 frames of 128x128x3, N=4096, MI355X\n")
    print("Command: `python tests/precision_study.py` (frames %s compared with the fp64 oracle).\n" % FRAMES)
    print("| storage | image max abs err | max err / max(|ref|, 1e-3) | max err in format spacings (|ref| >= 0.01) | "
          "grad shift from rounded dL/dI, median (x mag) | max (x mag) |")
    print("|---|---|---|---|---|---|")
    print("\n".join(rows))
    print("\n| storage | image MB | forward raster us | backward raster us |\n|---|---|---|---|")
    print("\n".join(times))


if __name__ == "__main__":
    main()
