"""Pins of the CPU oracle against mathematics it must satisfy (no GPU).

Each test fixes the oracle to something other than itself: closed-form
integrals and moments of a Gaussian, invariances of the parameterisation,
superposition, brute force on tiny inputs and central finite differences.
A plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed rotation, a mis-scaled exponent) fails at least one of them.
"""
import math

import numpy as np
import pytest

from differentiable_gaussian_splatting_pdr_amd import workloads


def one(mx, my, s1, s2, th, amps):
    return np.array([[[mx, my, s1, s2, th] + list(amps)]], dtype=np.float64)


def cov(s1, s2, th):
    # Sigma = R diag(s1^2, s2^2) R^T with axis 1 along (cos th, sin th)
    R = np.array([[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]])
    return R @ np.diag([s1 * s1, s2 * s2]) @ R.T


def grid(H, W):
    y, x = np.meshgrid(np.arange(H) + 0.5, np.arange(W) + 0.5, indexing="ij")
    return x, y


# untruncated kernels (k = 20) with s >= 1.5, mu >= 9 s from every border
CASES = [
    (1.5, 1.5, 0.0), (2.0, 5.0, 0.37), (6.0, 2.5, 1.1), (3.3, 1.7, 2.9), (7.0, 7.0, 0.8),
]


@pytest.mark.parametrize("s1,s2,th", CASES)
def test_integral_and_moments_untruncated(orc, s1, s2, th):
    H = W = 160
    mx, my, a = 80.3, 77.85, 1.7
    img, _, _, _ = orc.render(one(mx, my, s1, s2, th, [a]), H, W, radius=20.0)
    I = img[0, :, :, 0]
    x, y = grid(H, W)
    mass = a * 2 * math.pi * s1 * s2
    assert abs(I.sum() - mass) <= 1e-12 * mass
    # first moment = mass * mu
    assert abs((x * I).sum() - mass * mx) <= 1e-11 * mass * mx
    assert abs((y * I).sum() - mass * my) <= 1e-11 * mass * my
    # second central moment = mass * Sigma(theta); fixes the rotation sense
    S = cov(s1, s2, th)
    m2 = np.array([[((x - mx) ** 2 * I).sum(), ((x - mx) * (y - my) * I).sum()],
                   [((x - mx) * (y - my) * I).sum(), ((y - my) ** 2 * I).sum()]])
    assert np.abs(m2 - mass * S).max() <= 1e-9 * mass * np.trace(S)


def test_peak_is_amplitude_and_truncation_radius(orc):
    # pixel centre exactly at mu: w = 1; one pixel away along axis 1 of an
    # axis-aligned Gaussian: w = exp(-1/(2 s1^2)); beyond k sigma: 0
    a, s1, s2 = 2.5, 1.25, 0.8
    img, _, _, _ = orc.render(one(10.5, 7.5, s1, s2, 0.0, [a]), 16, 24, radius=3.0)
    I = img[0, :, :, 0]
    assert I[7, 10] == a
    assert abs(I[7, 11] - a * math.exp(-0.5 / s1 ** 2)) <= 1e-15 * a
    assert abs(I[8, 10] - a * math.exp(-0.5 / s2 ** 2)) <= 1e-15 * a
    assert abs(I[6, 12] - a * math.exp(-0.5 * (4 / s1 ** 2 + 1 / s2 ** 2))) <= 1e-15 * a
    # axis 1 extends 3*1.25 = 3.75 px: x offsets 3 kept, 4 dropped
    assert I[7, 13] > 0 and I[7, 14] == 0 and I[7, 7] > 0 and I[7, 6] == 0
    # axis 2 extends 3*0.8 = 2.4 px: y offsets 2 kept, 3 dropped
    assert I[9, 10] > 0 and I[10, 10] == 0


def test_truncation_edge_is_inclusive(orc):
    # axis-aligned s1 = s2 = 1 at a pixel centre: the pixel 3 px to the right
    # has q = 9 exactly; k = 3 keeps it (q <= k^2), k just below 3 drops it
    p = one(10.5, 10.5, 1.0, 1.0, 0.0, [1.0])
    for k, kept in ((3.0, True), (2.9997, False), (3.0003, True)):
        img, _, _, _ = orc.render(p, 21, 21, radius=k)
        assert (img[0, 10, 13, 0] == math.exp(-4.5)) == kept
        assert (img[0, 13, 10, 0] == math.exp(-4.5)) == kept
        assert img[0, 10, 14, 0] == 0.0
        # diagonal neighbour (2, 2): q = 8 < 9 always kept
        assert img[0, 12, 12, 0] == math.exp(-4.0)


@pytest.mark.parametrize("s", [1.0, 2.0, 4.0])
def test_truncated_integral(orc, s):
    # sum of a k-sigma truncated Gaussian ~ a 2 pi s1 s2 (1 - exp(-k^2/2));
    # the pixel grid discretises the edge, hence the loose bound
    H = W = 96
    k, a = 3.0, 1.0
    img, _, _, _ = orc.render(one(47.3, 51.1, s, 1.5 * s, 0.37, [a]), H, W, radius=k)
    want = a * 2 * math.pi * s * 1.5 * s * (1 - math.exp(-k * k / 2))
    assert abs(img.sum() - want) <= 5e-3 * want


def test_rotation_conventions(orc):
    H, W = 48, 56
    rng = np.random.default_rng(5)
    for _ in range(6):
        mx, my = rng.uniform(10, 46), rng.uniform(10, 38)
        s1, s2, th = rng.uniform(0.7, 4), rng.uniform(0.7, 4), rng.uniform(0, math.pi)
        a = [rng.normal(), rng.normal()]
        base, slk, _, _ = orc.render(one(mx, my, s1, s2, th, a), H, W, radius=3.0)
        for alt in (one(mx, my, s1, s2, th + math.pi, a), one(mx, my, s2, s1, th + math.pi / 2, a)):
            other, slk2, _, _ = orc.render(alt, H, W, radius=3.0)
            ok = (slk == 0) & (slk2 == 0)  # outside the truncation-tie band
            assert np.abs(other - base)[ok].max() <= 1e-13


def test_isotropic_independent_of_theta(orc):
    H = W = 40
    a = [1.3, -0.4, 2.0]
    ref, slk, _, _ = orc.render(one(19.2, 21.7, 2.2, 2.2, 0.0, a), H, W, radius=3.0)
    for th in (0.3, 1.0, 2.0, 3.0):
        img, slk2, _, _ = orc.render(one(19.2, 21.7, 2.2, 2.2, th, a), H, W, radius=3.0)
        ok = (slk == 0) & (slk2 == 0)
        assert np.abs(img - ref)[ok].max() <= 1e-14


def test_superposition_and_linearity(orc):
    p, _ = workloads.make_custom(2, 60, 37, 45, 3, seed=11)
    p = p.astype(np.float64)
    full, _, _, _ = orc.render(p, 37, 45)
    a, _, _, _ = orc.render(p[:, :23], 37, 45)
    b, _, _, _ = orc.render(p[:, 23:], 37, 45)
    assert np.abs(full - (a + b)).max() <= 1e-13
    q = p.copy()
    q[..., 5:] *= -2.5
    scaled, _, _, _ = orc.render(q, 37, 45)
    assert np.abs(scaled + 2.5 * full).max() <= 1e-13


def test_integer_shift_equivariance(orc):
    p = one(20.3, 18.9, 2.1, 3.4, 0.6, [1.0])
    img, _, _, _ = orc.render(p, 48, 48)
    p2 = p.copy()
    p2[0, 0, 0] += 5
    p2[0, 0, 1] += 3
    img2, _, _, _ = orc.render(p2, 48, 48)
    assert np.array_equal(img2[0, 3:, 5:], img[0, :-3, :-5])


def test_allpairs_equals_box_scatter(orc):
    # the box pruning changes nothing: every pixel x every Gaussian gives the
    # same image bit for bit (both add Gaussians in ascending order)
    _, p, _ = workloads.make_inputs(1, frames=3)
    a, sa, ma, pa = orc.render(p, 64, 64)
    b, sb, mb, pb = orc.render(p, 64, 64, allpairs=True)
    assert np.array_equal(a, b) and np.array_equal(sa, sb) and np.array_equal(pa, pb)
    p2, _ = workloads.make_custom(1, 40, 33, 29, 2, seed=3, s_range=(0.3, 9.0), mean_margin=15)
    a, _, _, _ = orc.render(p2, 33, 29)
    b, _, _, _ = orc.render(p2, 33, 29, allpairs=True)
    assert np.array_equal(a, b)


def test_support_count_matches_render(orc):
    _, p, _ = workloads.make_inputs(2, frames=3, with_grad=False)
    _, _, _, pairs = orc.render(p, 128, 128)
    assert np.array_equal(orc.count_support(p, 128, 128), pairs)
    p2, _ = workloads.make_custom(2, 40, 20, 30, 1, seed=9, mean_margin=5)
    img, _, _, pairs2 = orc.render(p2, 20, 30, allpairs=True)
    assert np.array_equal(orc.count_support(p2, 20, 30), pairs2)


def test_invalid_gaussians_are_culled(orc):
    p, g = workloads.make_custom(1, 8, 20, 20, 2, seed=2)
    p = p.astype(np.float64)
    ref, _, _, _ = orc.render(p[:, :4], 20, 20)
    bad = p.copy()
    bad[0, 4, 2] = 0.0
    bad[0, 5, 3] = -1.0
    bad[0, 6, 4] = np.nan
    bad[0, 7, 6] = np.inf
    img, _, _, _ = orc.render(bad, 20, 20)
    assert np.array_equal(img, ref)
    gr, _, _ = orc.grad(bad, g, 20, 20)
    assert np.all(gr[0, 4:] == 0)


# --- gradients ---------------------------------------------------------------

def _closed_grad(orc, G, p, H, W):
    gr, _, _ = orc.grad(p, G[None, :, :, None], H, W, radius=20.0)
    return gr[0, 0]


@pytest.mark.parametrize("s1,s2,th", [(2.0, 5.0, 0.37), (6.0, 2.5, 1.1), (3.0, 3.0, 2.2)])
def test_gradient_closed_forms(orc, s1, s2, th):
    H = W = 160
    mx, my, a = 80.3, 77.85, 1.7
    p = one(mx, my, s1, s2, th, [a])
    x, y = grid(H, W)
    tp = 2 * math.pi
    c, s = math.cos(th), math.sin(th)
    S = cov(s1, s2, th)
    sxx, syy, sxy = S[0, 0], S[1, 1], S[0, 1]
    tol = 1e-9

    def close(got, want, scale):
        assert abs(got - want) <= tol * scale, (got, want)

    # G = 1: L = a 2pi s1 s2
    g = _closed_grad(orc, np.ones((H, W)), p, H, W)
    sc = a * tp * s1 * s2
    close(g[5], tp * s1 * s2, sc)
    close(g[2], a * tp * s2, sc)
    close(g[3], a * tp * s1, sc)
    close(g[0], 0.0, sc)
    close(g[1], 0.0, sc)
    close(g[4], 0.0, sc)
    # G = p_x: L = a 2pi s1 s2 mu_x
    g = _closed_grad(orc, x, p, H, W)
    sc = a * tp * s1 * s2 * mx
    close(g[0], a * tp * s1 * s2, sc)
    close(g[1], 0.0, sc)
    close(g[2], a * tp * s2 * mx, sc)
    close(g[4], 0.0, sc)
    # G = (p_x - mu_x)^2: L = a 2pi s1 s2 Sigma_xx
    g = _closed_grad(orc, (x - mx) ** 2, p, H, W)
    sc = a * tp * s1 * s2 * (s1 * s1 + s2 * s2)
    close(g[0], 0.0, sc)
    close(g[4], a * tp * s1 * s2 * (s2 * s2 - s1 * s1) * math.sin(2 * th), sc)
    close(g[2], a * tp * s2 * (3 * s1 * s1 * c * c + s2 * s2 * s * s), sc)
    close(g[3], a * tp * s1 * (s1 * s1 * c * c + 3 * s2 * s2 * s * s), sc)
    close(g[5], tp * s1 * s2 * sxx, sc)
    # G = (p_y - mu_y)^2: L = a 2pi s1 s2 Sigma_yy
    g = _closed_grad(orc, (y - my) ** 2, p, H, W)
    close(g[1], 0.0, sc)
    close(g[4], a * tp * s1 * s2 * (s1 * s1 - s2 * s2) * math.sin(2 * th), sc)
    close(g[2], a * tp * s2 * (3 * s1 * s1 * s * s + s2 * s2 * c * c), sc)
    close(g[5], tp * s1 * s2 * syy, sc)
    # G = (p_x - mu_x)(p_y - mu_y): L = a 2pi s1 s2 Sigma_xy
    g = _closed_grad(orc, (x - mx) * (y - my), p, H, W)
    close(g[0], 0.0, sc)
    close(g[1], 0.0, sc)
    close(g[4], a * tp * s1 * s2 * (s1 * s1 - s2 * s2) * math.cos(2 * th), sc)
    close(g[2], a * tp * s2 * c * s * (3 * s1 * s1 - s2 * s2), sc)
    close(g[3], a * tp * s1 * c * s * (s1 * s1 - 3 * s2 * s2), sc)
    close(g[5], tp * s1 * s2 * sxy, sc)


def _loss(orc, p, G, H, W, k):
    img, _, _, _ = orc.render(p, H, W, radius=k, extras=False, nthreads=1)
    return float((img * G).sum())


@pytest.mark.parametrize("k", [20.0, 3.0])
def test_gradients_central_differences(orc, k):
    B, N, H, W, C = 2, 5, 24, 24, 2
    p, G = workloads.make_custom(B, N, H, W, C, seed=7, s_range=(0.8, 3.5), mean_margin=2.0)
    p = p.astype(np.float64)
    G = G.astype(np.float64)
    gr, _, _ = orc.grad(p, G, H, W, radius=k)
    # screen: with truncation, no pair may sit within 1e-3 k^2 of the edge
    _, band, _ = orc.grad(p, G, H, W, radius=k, tau=1e-3)
    checked = 0
    for b in range(B):
        for n in range(N):
            if k < 10 and np.any(band[b, n] != 0):
                continue
            for i in range(5 + C):
                h = 1e-6 * max(1.0, abs(p[b, n, i]))
                pp, pm = p.copy(), p.copy()
                pp[b, n, i] += h
                pm[b, n, i] -= h
                fd = (_loss(orc, pp, G, H, W, k) - _loss(orc, pm, G, H, W, k)) / (2 * h)
                scale = max(1.0, abs(gr[b, n, i]))
                assert abs(fd - gr[b, n, i]) <= 1e-6 * scale, (b, n, i, fd, gr[b, n, i])
                checked += 1
    assert checked >= 30


@pytest.mark.parametrize("k", [20.0, 3.0])
def test_gradients_adjoint(orc, k):
    # <G, J delta> by one central difference along delta == <J^T G, delta>
    _, p, G = workloads.make_inputs(2, frames=1)
    p = p.astype(np.float64)
    p = p[:, :512]
    H = W = 128
    gr, _, _ = orc.grad(p, G, H, W, radius=k)
    _, band, _ = orc.grad(p, G, H, W, radius=k, tau=1e-3)
    rng = np.random.default_rng(1)
    delta = rng.standard_normal(p.shape)
    delta[..., 2:4] *= 0.1 * p[..., 2:4]  # keep scales positive under the step
    if k < 10:
        delta[np.any(band != 0, axis=2)] = 0.0
    h = 1e-6
    fd = (_loss(orc, p + h * delta, G, H, W, k) - _loss(orc, p - h * delta, G, H, W, k)) / (2 * h)
    an = float((gr * delta).sum())
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (fd, an)


def test_slack_and_magnitude_bound_the_image(orc):
    _, p, G = workloads.make_inputs(0)
    img, slk, mag, _ = orc.render(p, 64, 64)
    assert np.all(slk >= 0) and np.all(mag >= np.abs(img))
    gr, gsl, gmag = orc.grad(p, G, 64, 64)
    assert np.all(gsl >= 0) and np.all(gmag >= np.abs(gr) * (1 - 1e-12))
    # tie slack only where a pair sits in the tie band: a tiny minority
    assert 0 < (slk > 0).sum() < 0.01 * slk.size
    assert (gsl > 0).sum() < 0.2 * gsl.size


def test_slack_is_exactly_the_tie_band_terms(orc):
    # the slack of a pixel is the sum of |a| w over the pairs with
    # |q - k^2| <= tau k^2 and nothing else: one isotropic Gaussian at a pixel
    # centre has pairs at q = 9 exactly (offsets (3, 0) ...), none within the
    # band otherwise
    a = -1.75
    p = one(10.5, 10.5, 1.0, 1.0, 0.0, [a])
    img, slk, mag, _ = orc.render(p, 21, 21, radius=3.0)
    want = np.zeros((21, 21))
    for dy in range(-4, 5):
        for dx in range(-4, 5):
            if abs(dx * dx + dy * dy - 9.0) <= 1e-4 * 9.0:
                want[10 + dy, 10 + dx] = abs(a) * math.exp(-4.5)
    assert np.array_equal(slk[0, :, :, 0], want)
    assert np.count_nonzero(want) == 4
    assert np.array_equal(mag[0, :, :, 0], np.abs(img[0, :, :, 0]))


# --- binning -------------------------------------------------------------------

def _boxes_numpy(p, H, W, k):
    """Pixel boxes from the covariance built as R diag R^T (another route)."""
    B, N, _ = p.shape
    out = np.full((B, N, 4), -1, np.int64)
    for b in range(B):
        for n in range(N):
            g = p[b, n]
            if not np.all(np.isfinite(g)) or g[2] <= 0 or g[3] <= 0:
                continue
            S = cov(g[2], g[3], g[4])
            ex, ey = k * math.sqrt(S[0, 0]), k * math.sqrt(S[1, 1])
            xs = [x for x in range(W) if abs(x + 0.5 - g[0]) <= ex]
            ys = [y for y in range(H) if abs(y + 0.5 - g[1]) <= ey]
            if xs and ys:
                out[b, n] = (xs[0], xs[-1], ys[0], ys[-1])
    return out


@pytest.mark.parametrize("shape", [(2, 70, 37, 53, 16), (1, 50, 64, 64, 16), (2, 40, 30, 20, 8)])
def test_binning_brute_force(orc, shape):
    B, N, H, W, T = shape
    p, _ = workloads.make_custom(B, N, H, W, 1, seed=N, s_range=(0.3, 7.0), mean_margin=12.0)
    p = p.astype(np.float64)
    p[0, 3, 2] = -1.0  # an invalid Gaussian is never listed
    counts, off, lst, rect = orc.bin(p, H, W, radius=3.0, tile=T)
    boxes = _boxes_numpy(p, H, W, 3.0)
    assert np.array_equal(rect, boxes)
    nTx, nTy = -(-W // T), -(-H // T)
    assert off[0] == 0 and np.array_equal(np.diff(off), counts.reshape(-1))
    for b in range(B):
        for ty in range(nTy):
            for tx in range(nTx):
                t = ty * nTx + tx
                seg = lst[off[b * nTx * nTy + t]:off[b * nTx * nTy + t + 1]]
                want = [n for n in range(N) if boxes[b, n, 0] >= 0
                        and boxes[b, n, 0] <= min(W - 1, tx * T + T - 1) and boxes[b, n, 1] >= tx * T
                        and boxes[b, n, 2] <= min(H - 1, ty * T + T - 1) and boxes[b, n, 3] >= ty * T]
                assert list(seg) == want


def test_support_lies_in_listed_tiles(orc):
    # every pixel with q <= k^2 (numpy, covariance route) is in a tile whose
    # list holds its Gaussian
    B, N, H, W, T = 1, 30, 45, 50, 16
    p, _ = workloads.make_custom(B, N, H, W, 1, seed=4, s_range=(0.4, 6.0), mean_margin=8.0)
    p = p.astype(np.float64)
    counts, off, lst, _ = orc.bin(p, H, W, radius=3.0, tile=T)
    nTx = -(-W // T)
    x, y = grid(H, W)
    for n in range(N):
        g = p[0, n]
        Si = np.linalg.inv(cov(g[2], g[3], g[4]))
        dx, dy = x - g[0], y - g[1]
        q = Si[0, 0] * dx * dx + 2 * Si[0, 1] * dx * dy + Si[1, 1] * dy * dy
        for yy, xx in zip(*np.nonzero(q <= 9.0 * (1 - 1e-9))):
            t = (yy // T) * nTx + (xx // T)
            assert n in lst[off[t]:off[t + 1]]


def test_binning_counts_on_workload(orc):
    # the list builder agrees with per-Gaussian boxes on a full-size frame
    _, p, _ = workloads.make_inputs(2, frames=2, with_grad=False)
    counts, off, lst, rect = orc.bin(p, 128, 128)
    area = np.where(rect[..., 0] >= 0,
                    (rect[..., 1] // 16 - rect[..., 0] // 16 + 1)
                    * (rect[..., 3] // 16 - rect[..., 2] // 16 + 1), 0)
    assert area.sum() == off[-1] == len(lst)


# --- the truncation-tie band ---------------------------------------------------------

def test_count_support_edge_is_inclusive(orc):
    # the support count uses the same inclusive edge as render: one isotropic
    # s = 1 Gaussian at a pixel centre has 29 pixel centres with
    # dx^2 + dy^2 <= 9 (4 of them at q = 9 exactly), 25 strictly inside
    p = one(10.5, 10.5, 1.0, 1.0, 0.0, [1.0])
    assert int(orc.count_support(p, 21, 21, 3.0)[0]) == 29
    assert int(orc.count_support(p, 21, 21, 2.9997)[0]) == 25
    assert int(orc.count_support(p, 21, 21, 3.0003)[0]) == 29
    # and by brute force over the lattice
    for k in (1.0, 2.5, 3.0, 4.0):
        n = sum(1 for dy in range(-6, 7) for dx in range(-6, 7) if dx * dx + dy * dy <= k * k)
        assert int(orc.count_support(p, 21, 21, k)[0]) == n


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_tie_band_exceeds_single_precision_q(orc, idx):
    # the reading behind the tie band: a pair within tau k^2 of the edge may
    # fall on either side in single precision.  For the workloads' Gaussians
    # (anisotropy up to 4:1, 10:1 and ~50:1) an fp32 evaluation of q from fp32
    # whitening rows and p - mu puts q within tau k^2 / 4 of the fp64 q on
    # every pixel of the box, so the band covers single-precision evaluation
    # of the definition with room to spare
    wl, p, _ = workloads.make_inputs(idx, frames=1, with_grad=False)
    k, tau = 3.0, 1e-4
    f = np.float32
    rng = np.random.default_rng(idx)
    g = p[0].astype(np.float64)
    s1, s2 = g[:, 2], g[:, 3]
    R = np.maximum(s1, s2) / np.minimum(s1, s2)
    sel = np.unique(np.concatenate([np.argsort(R)[-40:], rng.choice(len(g), 40, replace=False)]))
    worst = 0.0
    for n in sel:
        mx, my, a1, a2, th = g[n, :5]
        c, s = math.cos(th), math.sin(th)
        ex = k * math.hypot(a1 * c, a2 * s)
        ey = k * math.hypot(a1 * s, a2 * c)
        xs = np.arange(max(0, math.ceil(mx - ex - 0.5)), min(wl.W - 1, math.floor(mx + ex - 0.5)) + 1)
        ys = np.arange(max(0, math.ceil(my - ey - 0.5)), min(wl.H - 1, math.floor(my + ey - 0.5)) + 1)
        if xs.size == 0 or ys.size == 0:
            continue
        Y, X = np.meshgrid(ys + 0.5, xs + 0.5, indexing="ij")
        dx, dy = X - mx, Y - my
        q64 = ((c * dx + s * dy) / a1) ** 2 + ((-s * dx + c * dy) / a2) ** 2
        dxf, dyf = X.astype(f) - f(mx), Y.astype(f) - f(my)
        z1 = f(c / a1) * dxf + f(s / a1) * dyf
        z2 = f(-s / a2) * dxf + f(c / a2) * dyf
        q32 = (z1 * z1 + z2 * z2).astype(np.float64)
        m = q64 <= 2 * k * k
        if m.any():
            worst = max(worst, float(np.abs(q32 - q64)[m].max()))
    assert worst <= 0.25 * tau * k * k, worst
