"""Pins of the L1 + SSIM loss oracle (no GPU): the window against library
routines, SSIM(x, x) = 1, a closed form on constant frames, the L1 term, and
central finite differences of the whole loss."""
import math

import numpy as np
import pytest
import scipy.ndimage
import scipy.signal

from oracle import loss as ol


def test_window_matches_scipy():
    g = ol.window_1d()
    ref = scipy.signal.windows.gaussian(11, 1.5)
    assert np.allclose(g, ref / ref.sum(), rtol=0, atol=1e-16)
    assert abs(g.sum() - 1) < 1e-15


def test_window_sums_match_scipy_correlate():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((2, 13, 17, 3))
    g = ol.window_1d()
    out = ol._wsum(a, np.outer(g, g))
    for b in range(2):
        for c in range(3):
            ref = scipy.ndimage.correlate(a[b, :, :, c], np.outer(g, g), mode="constant", cval=0.0)
            assert np.abs(out[b, :, :, c] - ref).max() < 1e-14


def test_ssim_of_identical_frames_is_one():
    rng = np.random.default_rng(1)
    x = rng.uniform(0, 1, (2, 20, 23, 3))
    s, _ = ol.ssim_map(x, x)
    assert np.all(s == 1.0)
    loss, grad = ol.l1_ssim(x, x)
    assert loss == 0.0
    assert np.abs(grad).max() < 1e-15  # a maximum of SSIM, and sign(0) = 0


def test_ssim_closed_form_on_constant_frames():
    # away from the zero padding (5 px), every window sees constants a, b:
    # sigma terms vanish and s = (2ab + C1) / (a^2 + b^2 + C1)
    a, b = 0.7, 0.25
    x = np.full((1, 16, 18, 2), a)
    y = np.full((1, 16, 18, 2), b)
    s, _ = ol.ssim_map(x, y)
    want = (2 * a * b + ol.C1) / (a * a + b * b + ol.C1)
    assert np.abs(s[:, 5:-5, 5:-5, :] - want).max() < 1e-12


def test_ssim_map_against_scipy_route():
    # the same statistics from scipy's correlate, combined with the textbook
    # SSIM formula in terms of variances and covariance
    rng = np.random.default_rng(2)
    x = rng.uniform(0, 1, (1, 15, 14, 1))
    y = np.clip(x + 0.2 * rng.standard_normal(x.shape), 0, 1)
    g = ol.window_1d()
    w = np.outer(g, g)
    f = lambda a: scipy.ndimage.correlate(a, w, mode="constant", cval=0.0)
    X, Y = x[0, :, :, 0], y[0, :, :, 0]
    mx, my = f(X), f(Y)
    vx, vy, cxy = f(X * X) - mx * mx, f(Y * Y) - my * my, f(X * Y) - mx * my
    ref = ((2 * mx * my + ol.C1) * (2 * cxy + ol.C2)) / ((mx * mx + my * my + ol.C1) * (vx + vy + ol.C2))
    s, _ = ol.ssim_map(x, y)
    assert np.abs(s[0, :, :, 0] - ref).max() < 1e-12


def test_l1_term_alone():
    rng = np.random.default_rng(3)
    x, y = rng.standard_normal((2, 1, 9, 8, 2))
    loss, grad = ol.l1_ssim(x, y, lam=0.0)
    assert abs(loss - np.abs(x - y).mean()) < 1e-15
    assert np.array_equal(grad, np.sign(x - y) / x.size)


@pytest.mark.parametrize("lam", [0.2, 1.0])
def test_gradient_central_differences(lam):
    rng = np.random.default_rng(4)
    x = rng.uniform(0, 1, (2, 9, 10, 2))
    y = np.clip(x + rng.choice([-1, 1], x.shape) * rng.uniform(0.05, 0.3, x.shape), -1, 2)
    _, grad = ol.l1_ssim(x, y, lam=lam)
    h = 1e-6
    for idx in [(0, 0, 0, 0), (0, 4, 5, 1), (1, 8, 9, 0), (1, 2, 7, 1), (0, 6, 0, 1), (1, 0, 9, 0)]:
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd = (ol.l1_ssim(xp, y, lam=lam)[0] - ol.l1_ssim(xm, y, lam=lam)[0]) / (2 * h)
        assert abs(fd - grad[idx]) <= 1e-6 * abs(grad[idx]) + 1e-10, (idx, fd, grad[idx])


def test_ssim_symmetric_and_bounded():
    rng = np.random.default_rng(5)
    x = rng.uniform(0, 1, (1, 14, 12, 2))
    y = rng.uniform(0, 1, (1, 14, 12, 2))
    s1, _ = ol.ssim_map(x, y)
    s2, _ = ol.ssim_map(y, x)
    assert np.abs(s1 - s2).max() < 1e-15
    assert np.all(s1 <= 1.0) and np.all(s1 >= -1.0)


def test_gradient_magnitude_bounds_gradient():
    rng = np.random.default_rng(6)
    x = rng.uniform(0, 1, (1, 12, 13, 3))
    y = np.clip(x + 0.1 * rng.standard_normal(x.shape), 0, 1)
    _, g, mag = ol.l1_ssim(x, y, with_mag=True)
    assert np.all(np.abs(g) <= mag * (1 + 1e-12))
    assert np.all(mag > 0)
