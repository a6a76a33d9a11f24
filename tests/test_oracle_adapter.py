"""Pins of the adapter-side oracle (no GPU): grid centres by hand, grid
initialisation through the activation, the activation's bounds, its
gradient against central differences, concat and its adjoint, and an
end-to-end identity through the renderer oracle."""
import numpy as np
import pytest

import oracle
from oracle import adapter as oa


def test_grid_centres_by_hand():
    g, (cw, ch) = oa.grid_centres(4, 2, 8, 16)   # 16 wide, 8 tall: 4 x 4 cells
    assert (cw, ch) == (4.0, 4.0)
    want = [(2, 2), (6, 2), (10, 2), (14, 2), (2, 6), (6, 6), (10, 6), (14, 6)]
    assert np.array_equal(g, np.array(want, float))
    g, (cw, ch) = oa.grid_centres(3, 5, 10, 9)    # non-square cells 3 x 2
    assert (cw, ch) == (3.0, 2.0)
    assert np.array_equal(g[7], [4.5, 5.0])       # i = 1, j = 2


def test_grid_init_activates_onto_the_grid():
    B, gx, gy, H, W, C = 2, 3, 2, 6, 9, 2
    img = np.arange(B * H * W * C, dtype=np.float64).reshape(B, H, W, C)
    raw = oa.grid_init(B, gx, gy, H, W, C, 0.5, image=img)
    p = oa.activate(raw, gx, gy, H, W)
    # cells are 3 x 3; centres (1.5, 1.5), (4.5, 1.5), ..., pixel (1, 1), (4, 1), ...
    assert np.array_equal(p[0, :, 0], [1.5, 4.5, 7.5, 1.5, 4.5, 7.5])
    assert np.array_equal(p[0, :, 1], [1.5, 1.5, 1.5, 4.5, 4.5, 4.5])
    assert np.allclose(p[..., 2], 1.5, rtol=1e-15) and np.allclose(p[..., 3], 1.5, rtol=1e-15)
    assert np.all(p[..., 4] == 0)
    for b in range(B):
        for n, (x, y) in enumerate([(1, 1), (4, 1), (7, 1), (1, 4), (4, 4), (7, 4)]):
            assert np.array_equal(p[b, n, 5:], img[b, y, x])
    assert np.all(oa.grid_init(1, gx, gy, H, W, C, 0.5)[..., 5:] == 0)


def test_activation_bounds():
    rng = np.random.default_rng(0)
    gx, gy, H, W = 5, 3, 30, 40
    raw = 5 * rng.standard_normal((2, gx * gy, 8))
    p = oa.activate(raw, gx, gy, H, W)
    g, (cw, ch) = oa.grid_centres(gx, gy, H, W)
    assert np.all(np.abs(p[..., 0] - g[:, 0]) <= cw) and np.all(np.abs(p[..., 1] - g[:, 1]) <= ch)
    assert np.all(p[..., 2] > 0) and np.all(p[..., 3] > 0)
    assert np.array_equal(p[..., 4:], raw[..., 4:])


def test_activation_backward_central_differences():
    rng = np.random.default_rng(1)
    gx, gy, H, W, C = 3, 2, 10, 12, 2
    raw = rng.standard_normal((2, gx * gy, 5 + C))
    G = rng.standard_normal(raw.shape)
    gr = oa.activate_backward(raw, G, gx, gy, H, W)
    h = 1e-6
    for idx in [(0, 0, 0), (0, 3, 1), (1, 5, 2), (1, 2, 3), (0, 4, 4), (1, 1, 6)]:
        rp, rm = raw.copy(), raw.copy()
        rp[idx] += h
        rm[idx] -= h
        fd = ((oa.activate(rp, gx, gy, H, W) - oa.activate(rm, gx, gy, H, W)) * G).sum() / (2 * h)
        assert abs(fd - gr[idx]) <= 1e-8 * max(1.0, abs(gr[idx])), (idx, fd, gr[idx])


def test_concat_and_adjoint():
    rng = np.random.default_rng(2)
    pix = rng.standard_normal((2, 4, 5, 2))
    ren = rng.standard_normal((2, 4, 5, 3))
    out = oa.concat(pix, ren)
    assert out.shape == (2, 4, 5, 5)
    assert np.array_equal(out[..., 0], pix[..., 0]) and np.array_equal(out[..., 4], ren[..., 2])
    G = rng.standard_normal(out.shape)
    gp, gr = oa.concat_backward(G, 2)
    lhs = (out * G).sum()
    rhs = (pix * gp).sum() + (ren * gr).sum()
    assert abs(lhs - rhs) <= 1e-12 * abs(lhs)


def test_one_gaussian_per_pixel_reproduces_the_frame(orc):
    # a Gaussian on every pixel centre with s = 0.3 px: its 3-sigma support
    # (0.9 px) holds its own pixel centre only, with weight exp(0) = 1
    rng = np.random.default_rng(3)
    B, H, W, C = 2, 6, 7, 2
    img = rng.standard_normal((B, H, W, C))
    raw = oa.grid_init(B, W, H, H, W, C, 0.3, image=img)
    p = oa.activate(raw, W, H, H, W).astype(np.float32)
    out, _, _, _ = oracle.render(p, H, W, 3.0)
    assert np.abs(out - img.astype(np.float32)).max() < 1e-6
