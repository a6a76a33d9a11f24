"""fp64 oracle of the plain adapter-side operations around the renderer.

TEST INFRASTRUCTURE ONLY (imported by tests/).

Page 2 of the sources (the reading notes on "Learning Video Dynamics with
Predictive Differentiable Rendering", section "Method") says the PredGS
adapter regresses the Gaussian parameters from the backbone's coarse
prediction, and its section "Relation To Prior Work" names grid
initialisation and concat fusion of the pixel and Gaussian branches as
parts of the design; page 1 (Abstract) fixes the 5 + C parameters.  The
pages give no formula for any of them; the readings taken here (listed in
the design notes) are the plainest ones:

Grid.  N = gx * gy Gaussians per frame, n = j * gx + i (row-major), cell
size (cw, ch) = (W / gx, H / gy), centre g_n = ((i + 1/2) cw, (j + 1/2) ch).

Activation (raw adapter output r -> renderer parameters):
    mu_x = g_x + cw * tanh(r0)        mu_y = g_y + ch * tanh(r1)
    s1   = cw * exp(r2)               s2   = ch * exp(r3)
    theta = r4                        a_c  = r_{5+c}
so a Gaussian stays within one cell of its grid centre and its scales are
positive multiples of the cell size.

Grid initialisation: the raw values r = (0, 0, ln s0, ln s0, 0, a) whose
activation puts every Gaussian on its grid centre with scales s0 * cell,
theta = 0, and amplitudes a_c sampled from an optional coarse frame at the
pixel that contains the centre (0 without one).

Concat fusion: out[..., :Cp] = the pixel-branch frame, out[..., Cp:] = the
rendered frame; its gradient splits the same way.
"""
from __future__ import annotations

import numpy as np


def grid_centres(gx, gy, H, W):
    """(N, 2) fp64 centres and the cell size (cw, ch)."""
    cw, ch = W / gx, H / gy
    j, i = np.divmod(np.arange(gx * gy), gx)
    return np.stack([(i + 0.5) * cw, (j + 0.5) * ch], axis=1), (cw, ch)


def grid_init(B, gx, gy, H, W, C, s0, image=None):
    """Raw parameters [B][gx*gy][5+C] (fp64)."""
    N = gx * gy
    raw = np.zeros((B, N, 5 + C), np.float64)
    raw[..., 2] = np.log(s0)
    raw[..., 3] = np.log(s0)
    if image is not None:
        # the pixel containing the centre, floor((2i + 1) W / (2 gx)), in
        # exact integer arithmetic
        j, i = np.divmod(np.arange(N), gx)
        px = ((2 * i + 1) * W) // (2 * gx)
        py = ((2 * j + 1) * H) // (2 * gy)
        raw[..., 5:] = np.asarray(image, np.float64)[:, py, px, :]
    return raw


def activate(raw, gx, gy, H, W):
    r = np.asarray(raw, np.float64)
    g, (cw, ch) = grid_centres(gx, gy, H, W)
    p = np.empty_like(r)
    p[..., 0] = g[:, 0] + cw * np.tanh(r[..., 0])
    p[..., 1] = g[:, 1] + ch * np.tanh(r[..., 1])
    p[..., 2] = cw * np.exp(r[..., 2])
    p[..., 3] = ch * np.exp(r[..., 3])
    p[..., 4] = r[..., 4]
    p[..., 5:] = r[..., 5:]
    return p


def activate_backward(raw, grad_params, gx, gy, H, W):
    """dL/draw from dL/dparams: the derivative of each activation above."""
    r = np.asarray(raw, np.float64)
    gp = np.asarray(grad_params, np.float64)
    _, (cw, ch) = grid_centres(gx, gy, H, W)
    out = np.array(gp, np.float64)
    # d tanh(r)/dr = sech^2 r, written 1 / cosh^2 r (no cancellation at large |r|)
    out[..., 0] = gp[..., 0] * cw / np.cosh(r[..., 0]) ** 2
    out[..., 1] = gp[..., 1] * ch / np.cosh(r[..., 1]) ** 2
    out[..., 2] = gp[..., 2] * cw * np.exp(r[..., 2])
    out[..., 3] = gp[..., 3] * ch * np.exp(r[..., 3])
    return out


def concat(pixel, rendered):
    """Channel concatenation [B,H,W,Cp] + [B,H,W,C] -> [B,H,W,Cp+C]."""
    return np.concatenate([np.asarray(pixel), np.asarray(rendered)], axis=-1)


def concat_backward(grad_out, Cp):
    g = np.asarray(grad_out)
    return g[..., :Cp], g[..., Cp:]
