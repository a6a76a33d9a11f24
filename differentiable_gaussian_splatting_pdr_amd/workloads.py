"""Seeded synthetic inputs for the 2D Gaussian splatting layer.

This module only draws random numbers; it holds none of the renderer's
arithmetic.  Both the HIP path (through the tests and the benchmark) and the
CPU oracle consume exactly the fp32 arrays produced here.

Parameter layout per Gaussian (the abstract of "Learning Video Dynamics with
Predictive Differentiable Rendering" gives 5 + C learnable values: position,
scale, rotation and C channel amplitudes):

    [mu_x, mu_y, s1, s2, theta, a_0 .. a_{C-1}]

with mu in pixel units (x to the right, y down, pixel (x, y) covers
[x, x+1) x [y, y+1)), s1/s2 per-axis standard deviations in pixels and theta
the angle of axis 1 in radians.

Workloads (B frames, H x W x C grid, N Gaussians per frame):

  0  B=1,   64x64x1,    N=256,   means U[0,64)^2, s iid log-U[0.5,4], a~N(0,1)
  1  B=160, 64x64x1,    N=1024,  same distributions (video-prediction shape)
  2  B=384, 128x128x3,  N=4096,  s1 log-U[0.5,8], s2 log-U within 4:1 of s1,
                                  a~N(0,0.5) per channel
  3  B=192, 128x256x16, N=8192,  s1 log-U[1,12], s2 log-U within 10:1 of s1,
                                  a~N(0,1) with each (n,c) zeroed w.p. 0.3
  4  B=80,  512x512x3,  N=65536, means from a 32-centre isotropic mixture
                                  (sigma 20 px, centres U[0,512)^2, not
                                  clipped), s iid exp(N(ln 2, 0.8)) clipped to
                                  [0.3, 64], a~N(0,0.3)

theta ~ U[0, pi) and dL/dI ~ N(0, 1) everywhere; truncation radius 3 sigma.
Random draws use numpy's default_rng(seed) (PCG64), seed = workload index
unless given, drawn in fp64 and cast to fp32, in a fixed order per frame:
means, s1, s2, theta, amplitudes, zero-mask; then dL/dI for the whole batch.
"""
from __future__ import annotations

import dataclasses

import numpy as np

RADIUS = 3.0


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    B: int
    H: int
    W: int
    C: int
    N: int
    desc: str

    @property
    def name(self) -> str:
        return f"cfg{self.index}:B{self.B}x{self.H}x{self.W}x{self.C}/N{self.N}"


WORKLOADS = (
    Workload(0, 1, 64, 64, 1, 256, "single 64x64 frame, C=1, N=256"),
    Workload(1, 160, 64, 64, 1, 1024, "16x10 frames, 64x64, C=1, N=1024"),
    Workload(2, 384, 128, 128, 3, 4096, "32x12 frames, 128x128x3, N=4096"),
    Workload(3, 192, 128, 256, 16, 8192, "16x12 frames, 128x256x16, N=8192"),
    Workload(4, 80, 512, 512, 3, 65536, "8x10 frames, 512x512x3, N=65536, clustered"),
)


def _log_uniform(rng, lo, hi, size=None):
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=size))


def _draw_frame(rng, idx, N, H, W, C):
    """One frame's Gaussians as an fp64 [N, 5 + C] array."""
    p = np.empty((N, 5 + C), dtype=np.float64)
    if idx in (0, 1, 2, 3):
        p[:, 0] = rng.uniform(0.0, W, size=N)
        p[:, 1] = rng.uniform(0.0, H, size=N)
    else:
        centres = rng.uniform(0.0, [W, H], size=(32, 2))
        comp = rng.integers(0, 32, size=N)
        p[:, 0:2] = centres[comp] + 20.0 * rng.standard_normal(size=(N, 2))
    if idx in (0, 1):
        p[:, 2] = _log_uniform(rng, 0.5, 4.0, N)
        p[:, 3] = _log_uniform(rng, 0.5, 4.0, N)
    elif idx == 2:
        s1 = _log_uniform(rng, 0.5, 8.0, N)
        p[:, 2] = s1
        p[:, 3] = _log_uniform(rng, np.maximum(0.5, s1 / 4.0), np.minimum(8.0, 4.0 * s1))
    elif idx == 3:
        s1 = _log_uniform(rng, 1.0, 12.0, N)
        p[:, 2] = s1
        p[:, 3] = _log_uniform(rng, np.maximum(1.0, s1 / 10.0), np.minimum(12.0, 10.0 * s1))
    else:
        p[:, 2] = np.clip(np.exp(rng.normal(np.log(2.0), 0.8, size=N)), 0.3, 64.0)
        p[:, 3] = np.clip(np.exp(rng.normal(np.log(2.0), 0.8, size=N)), 0.3, 64.0)
    p[:, 4] = rng.uniform(0.0, np.pi, size=N)
    amp_std = {0: 1.0, 1: 1.0, 2: 0.5, 3: 1.0, 4: 0.3}[idx]
    p[:, 5:] = amp_std * rng.standard_normal(size=(N, C))
    if idx == 3:
        p[:, 5:] *= rng.uniform(size=(N, C)) >= 0.3
    return p


def make_inputs(index: int, frames: int | None = None, seed: int | None = None,
                with_grad: bool = True):
    """Return (workload, params f32[B,N,5+C], grad_image f32[B,H,W,C] or None).

    ``frames`` truncates the batch to its first frames (same draws for those
    frames as the full batch), for small-size tests.
    """
    wl = WORKLOADS[index]
    B = wl.B if frames is None else int(frames)
    rng = np.random.default_rng(index if seed is None else seed)
    params = np.empty((B, wl.N, 5 + wl.C), dtype=np.float32)
    for b in range(B):
        params[b] = _draw_frame(rng, index, wl.N, wl.H, wl.W, wl.C)
    grad = None
    if with_grad:
        grad = rng.standard_normal(size=(B, wl.H, wl.W, wl.C), dtype=np.float32)
    return dataclasses.replace(wl, B=B), params, grad


def make_custom(B: int, N: int, H: int, W: int, C: int, seed: int,
                s_range=(0.5, 6.0), mean_margin: float = 0.0, amp_std: float = 1.0):
    """Generic seeded inputs for edge-case and ragged-shape tests.

    Means are U[-margin, W+margin) x U[-margin, H+margin), scales iid
    log-uniform in ``s_range``, theta U[0, pi), amplitudes N(0, amp_std),
    dL/dI N(0, 1).
    """
    rng = np.random.default_rng(seed)
    p = np.empty((B, N, 5 + C), dtype=np.float64)
    p[..., 0] = rng.uniform(-mean_margin, W + mean_margin, size=(B, N))
    p[..., 1] = rng.uniform(-mean_margin, H + mean_margin, size=(B, N))
    p[..., 2] = _log_uniform(rng, s_range[0], s_range[1], (B, N))
    p[..., 3] = _log_uniform(rng, s_range[0], s_range[1], (B, N))
    p[..., 4] = rng.uniform(0.0, np.pi, size=(B, N))
    p[..., 5:] = amp_std * rng.standard_normal(size=(B, N, C))
    grad = rng.standard_normal(size=(B, H, W, C), dtype=np.float32)
    return p.astype(np.float32), grad


def make_loss_inputs(B: int, H: int, W: int, C: int, seed: int, kind: str = "noisy"):
    """Seeded (image, target) pairs in [0, 1]-like ranges for the training loss.

    "noisy": target ~ U[0, 1], image = target + N(0, 0.1);
    "flat":  target = 0.5 + N(0, 0.01), image = target + N(0, 0.005) (small
             local variances, the hard case for single-precision moments).
    """
    rng = np.random.default_rng(seed)
    if kind == "noisy":
        t = rng.uniform(0.0, 1.0, size=(B, H, W, C))
        x = t + 0.1 * rng.standard_normal(size=(B, H, W, C))
    elif kind == "flat":
        t = 0.5 + 0.01 * rng.standard_normal(size=(B, H, W, C))
        x = t + 0.005 * rng.standard_normal(size=(B, H, W, C))
    else:
        raise ValueError(kind)
    return x.astype(np.float32), t.astype(np.float32)
