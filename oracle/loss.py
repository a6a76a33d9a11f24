"""fp64 oracle of the combined L1 + SSIM training loss and its gradient.

TEST INFRASTRUCTURE ONLY (imported by tests/ and the benchmark's CPU leg).

The abstract of "Learning Video Dynamics with Predictive Differentiable
Rendering" says the model is optimised by a combined L1 and SSIM loss, and
the reading notes (section "Method") call L1 + SSIM necessary.  Neither page
gives the weighting or the SSIM window, so this module takes the plainest
readings (listed in the design notes):

  loss = (1 - lam) * mean |I - T| + lam * (1 - mean SSIM(I, T))

with lam = 0.2 by default, SSIM computed per frame and channel with the
standard 11 x 11 Gaussian window of sigma 1.5 (weights normalised to sum 1),
zero padding outside the frame ("same" size), C1 = 0.01^2, C2 = 0.03^2, and
the mean taken over all B*H*W*C pixels.  d|u|/du at u = 0 is taken as 0.

Everything here is the definition written out with numpy: window sums are
explicit shifted sums over the 121 window offsets (no separability), and
the gradient is the chain rule through the five window moments:

  mu_x = G*x, mu_y = G*y, m_xx = G*x^2, m_yy = G*y^2, m_xy = G*(xy)
  A1 = 2 mu_x mu_y + C1,  A2 = 2 (m_xy - mu_x mu_y) + C2
  B1 = mu_x^2 + mu_y^2 + C1,  B2 = (m_xx - mu_x^2) + (m_yy - mu_y^2) + C2
  s = A1 A2 / (B1 B2)
  ds/dmu_x = 2 mu_y (A2 - A1) / (B1 B2) - 2 mu_x s (1/B1 - 1/B2)
  ds/dm_xx = -s / B2,   ds/dm_xy = 2 A1 / (B1 B2)
  d mean(s) / dx(q) = (1/M) [ (G (x) ds/dmu_x)(q) + 2 x(q) (G (x) ds/dm_xx)(q)
                              + y(q) (G (x) ds/dm_xy)(q) ]

where (x) correlates with the window over pixels inside the frame.
"""
from __future__ import annotations

import math

import numpy as np

WIN = 11
SIGMA = 1.5
C1 = 0.01 ** 2
C2 = 0.03 ** 2
LAMBDA = 0.2


def window_1d(win=WIN, sigma=SIGMA):
    k = np.arange(win) - win // 2
    g = np.exp(-(k * k) / (2.0 * sigma * sigma))
    return g / g.sum()


def _wsum(a, g2):
    """Window sum with zero padding: out[y,x] = sum_{i,j} g2[i,j] a[y+i-r, x+j-r]
    over [B,H,W,C] arrays (the window is symmetric, so this is also the
    correlation used by the gradient)."""
    B, H, W, C = a.shape
    r = g2.shape[0] // 2
    pad = np.zeros((B, H + 2 * r, W + 2 * r, C), np.float64)
    pad[:, r:r + H, r:r + W, :] = a
    out = np.zeros_like(a, dtype=np.float64)
    for i in range(g2.shape[0]):
        for j in range(g2.shape[1]):
            out += g2[i, j] * pad[:, i:i + H, j:j + W, :]
    return out


def ssim_map(x, y, c1=C1, c2=C2, win=WIN, sigma=SIGMA):
    """Per-pixel SSIM s and the window moments (fp64)."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    g = window_1d(win, sigma)
    g2 = np.outer(g, g)
    mx, my = _wsum(x, g2), _wsum(y, g2)
    mxx, myy, mxy = _wsum(x * x, g2), _wsum(y * y, g2), _wsum(x * y, g2)
    a1 = 2 * mx * my + c1
    a2 = 2 * (mxy - mx * my) + c2
    b1 = mx * mx + my * my + c1
    b2 = (mxx - mx * mx) + (myy - my * my) + c2
    s = a1 * a2 / (b1 * b2)
    return s, dict(mx=mx, my=my, a1=a1, a2=a2, b1=b1, b2=b2, g2=g2)


def l1_ssim(image, target, lam=LAMBDA, c1=C1, c2=C2, win=WIN, sigma=SIGMA, with_mag=False):
    """Return (loss, dloss/dimage) in fp64 for [B,H,W,C] arrays; with_mag adds
    the per-value magnitude (sum of the absolute values of the gradient's
    terms), the scale its rounding error refers to."""
    x = np.asarray(image, np.float64)
    y = np.asarray(target, np.float64)
    M = x.size
    s, m = ssim_map(x, y, c1, c2, win, sigma)
    loss = (1 - lam) * np.abs(x - y).mean() + lam * (1 - s.mean())
    bb = m["b1"] * m["b2"]
    d_mu = 2 * m["my"] * (m["a2"] - m["a1"]) / bb - 2 * m["mx"] * s * (1 / m["b1"] - 1 / m["b2"])
    d_xx = -s / m["b2"]
    d_xy = 2 * m["a1"] / bb
    g2 = m["g2"]
    dssim = (_wsum(d_mu, g2) + 2 * x * _wsum(d_xx, g2) + y * _wsum(d_xy, g2)) / M
    grad = (1 - lam) * np.sign(x - y) / M - lam * dssim
    if not with_mag:
        return float(loss), grad
    mag = ((1 - lam) * np.abs(np.sign(x - y)) + lam * (
        _wsum(np.abs(d_mu), g2) + 2 * np.abs(x) * _wsum(np.abs(d_xx), g2)
        + np.abs(y) * _wsum(np.abs(d_xy), g2))) / M
    return float(loss), grad, mag
