"""HIP adapter-side ops (grid initialisation, activation and its gradient,
concat fusion of the renderer's output) against the fp64 oracle, on the GPU.

Tolerances: grid initialisation copies values (bit-exact) except ln(s0),
within 2 fp32 ulp; the activation and its gradient are evaluated in fp32
transcendental functions and combined in fp64, so each value is within
1e-6 of its scale (|ref| plus the cell size for the means); concat copies
are bit-exact, and the rendered part and the gradients meet the renderer's
tolerance (helpers.check_close)."""
import numpy as np
import pytest

from differentiable_gaussian_splatting_pdr_amd import workloads
from oracle import adapter as oa
from helpers import check_grad, check_close

pytestmark = pytest.mark.gpu


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


@pytest.mark.parametrize("B,gx,gy,H,W,C,s0", [
    (2, 4, 3, 16, 24, 3, 0.5), (1, 7, 5, 37, 53, 1, 0.3), (3, 64, 64, 128, 128, 3, 0.5),
    (1, 10, 3, 9, 31, 16, 1.25), (1, 1, 1, 1, 1, 1, 2.0),
])
def test_grid_init(B, gx, gy, H, W, C, s0):
    torch, dev = torch_dev()
    from differentiable_gaussian_splatting_pdr_amd import splat
    rng = np.random.default_rng(B * 1000 + gx)
    img = rng.standard_normal((B, H, W, C)).astype(np.float32)
    raw = splat.grid_init(B, gx, gy, H, W, C, s0, image=torch.from_numpy(img).to(dev)).cpu().numpy()
    ref = oa.grid_init(B, gx, gy, H, W, C, s0, image=img)
    assert np.array_equal(raw[..., [0, 1, 4]], ref[..., [0, 1, 4]])
    assert np.array_equal(raw[..., 5:], ref[..., 5:].astype(np.float32))
    assert np.all(np.abs(raw[..., 2:4] - ref[..., 2:4]) <= 2 * np.spacing(np.float32(abs(np.log(s0)) + 1e-30)))
    raw0 = splat.grid_init(B, gx, gy, H, W, C, s0, device=dev).cpu().numpy()
    assert np.all(raw0[..., 5:] == 0)


def _raw(B, N, C, seed, scale=1.5):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((B, N, 5 + C))).astype(np.float32)


@pytest.mark.parametrize("B,gx,gy,H,W,C", [
    (2, 4, 3, 16, 24, 3), (1, 7, 5, 37, 53, 1), (384, 64, 64, 128, 128, 3), (1, 11, 13, 100, 90, 20),
])
def test_activation_and_gradient(B, gx, gy, H, W, C):
    torch, dev = torch_dev()
    from differentiable_gaussian_splatting_pdr_amd import splat
    raw = _raw(B, gx * gy, C, seed=gx * gy + C)
    G = _raw(B, gx * gy, C, seed=7, scale=1.0)
    rt = torch.from_numpy(raw).to(dev).requires_grad_(True)
    p = splat.activate(rt, gx, gy, H, W)
    p.backward(torch.from_numpy(G).to(dev))
    got, gg = p.detach().cpu().numpy(), rt.grad.cpu().numpy()
    ref = oa.activate(raw, gx, gy, H, W)
    gref = oa.activate_backward(raw, G, gx, gy, H, W)
    _, (cw, ch) = oa.grid_centres(gx, gy, H, W)
    scale = np.abs(ref)
    scale[..., 0] += cw
    scale[..., 1] += ch
    assert np.all(np.abs(got - ref) <= 1e-6 * scale + 1e-30)
    assert np.array_equal(got[..., 4:], raw[..., 4:])
    assert np.all(np.abs(gg - gref) <= 1e-6 * np.abs(gref) + 1e-30)
    assert np.array_equal(gg[..., 4:], G[..., 4:])


def test_one_gaussian_per_pixel_reproduces_the_frame():
    torch, dev = torch_dev()
    from differentiable_gaussian_splatting_pdr_amd import splat
    B, H, W, C = 2, 24, 40, 3
    img = np.random.default_rng(9).standard_normal((B, H, W, C)).astype(np.float32)
    raw = splat.grid_init(B, W, H, H, W, C, 0.3, image=torch.from_numpy(img).to(dev))
    params = splat.activate(raw, W, H, H, W)
    out = splat.render(params, H, W).cpu().numpy()
    assert np.abs(out - img).max() <= 1e-6 * np.abs(img).max()


@pytest.mark.parametrize("case", [
    dict(B=2, N=60, H=37, W=53, C=3, Cp=2), dict(B=1, N=40, H=20, W=33, C=20, Cp=5),
    dict(B=3, N=30, H=16, W=16, C=1, Cp=1),
])
def test_concat_fusion(orc, case):
    torch, dev = torch_dev()
    from differentiable_gaussian_splatting_pdr_amd import splat
    B, N, H, W, C, Cp = (case[k] for k in ("B", "N", "H", "W", "C", "Cp"))
    params, _ = workloads.make_custom(B, N, H, W, C, seed=B * N + Cp)
    rng = np.random.default_rng(Cp)
    pix = rng.standard_normal((B, H, W, Cp)).astype(np.float32)
    gout = rng.standard_normal((B, H, W, Cp + C)).astype(np.float32)
    pt = torch.from_numpy(params).to(dev).requires_grad_(True)
    xt = torch.from_numpy(pix).to(dev).requires_grad_(True)
    out = splat.render_concat(pt, xt, H, W)
    out.backward(torch.from_numpy(gout).to(dev))
    o = out.detach().cpu().numpy()
    assert np.array_equal(o[..., :Cp], pix)
    img, slk, _, _ = orc.render(params, H, W, 3.0)
    check_close(o[..., Cp:], img, np.abs(img), slk, "rendered part")
    gr, gsl, gmag = orc.grad(params, np.ascontiguousarray(gout[..., Cp:]), H, W, 3.0)
    check_grad(pt.grad.cpu().numpy(), gr, gmag, gsl, "grad params")
    assert np.array_equal(xt.grad.cpu().numpy(), gout[..., :Cp])
    # the plain entry point on the same inputs gives the same rendered bits
    plain, _ = splat.forward(pt.detach(), H, W)
    assert np.array_equal(plain.cpu().numpy(), o[..., Cp:])


def test_concat_benchmark_shape_sampled_frames(orc):
    torch, dev = torch_dev()
    from differentiable_gaussian_splatting_pdr_amd import splat
    wl, params, grad = workloads.make_inputs(2)
    B, H, W, C, Cp = wl.B, wl.H, wl.W, wl.C, 3
    pix = np.random.default_rng(11).standard_normal((B, H, W, Cp)).astype(np.float32)
    gout = np.concatenate([np.random.default_rng(12).standard_normal((B, H, W, Cp)).astype(np.float32),
                           grad], axis=-1)
    pt = torch.from_numpy(params).to(dev)
    out, ws = splat.forward_concat(pt, torch.from_numpy(pix).to(dev), H, W)
    gp, gx = splat.backward_concat(pt, torch.from_numpy(gout).to(dev), Cp, H, W, workspace=ws,
                                   reuse_binning=True)
    o, gp, gx = out.cpu().numpy(), gp.cpu().numpy(), gx.cpu().numpy()
    assert np.array_equal(o[..., :Cp], pix) and np.array_equal(gx, gout[..., :Cp])
    for f in (0, 200, 383):
        img, slk, _, _ = orc.render(params[f:f + 1], H, W, 3.0)
        check_close(o[f:f + 1, ..., Cp:], img, np.abs(img), slk, "frame %d" % f)
        gr, gsl, gmag = orc.grad(params[f:f + 1], grad[f:f + 1], H, W, 3.0)
        check_grad(gp[f:f + 1], gr, gmag, gsl, "grad frame %d" % f)


def test_adapter_render_loss_chain(orc):
    """The whole training chain of the layer through autograd: raw adapter
    output -> activate -> render -> L1 + SSIM loss -> d loss / d raw, against
    the fp64 oracle composed step by step (activation, render, loss gradient,
    render backward, activation backward).  The activation's Jacobian is
    diagonal, so the renderer's bound carries over scaled by it; the factor
    1e-3 on the magnitude (ten times the renderer's) covers the loss
    gradient's own fp32 error propagated through the render backward."""
    torch, dev = torch_dev()
    from differentiable_gaussian_splatting_pdr_amd import splat
    from oracle import loss as ol
    B, gx, gy, H, W, C = 2, 12, 10, 45, 52, 3
    r0 = splat.grid_init(B, gx, gy, H, W, C, 0.5, device=dev)
    assert tuple(r0.shape) == (B, gx * gy, 5 + C)
    rng = np.random.default_rng(2024)
    raw = np.zeros((B, gx * gy, 5 + C))
    raw[..., 0:2] = 0.5 * rng.standard_normal((B, gx * gy, 2))
    raw[..., 2:4] = np.log(0.5) + 0.3 * rng.standard_normal((B, gx * gy, 2))
    raw[..., 4] = rng.uniform(-np.pi, np.pi, (B, gx * gy))
    raw[..., 5:] = rng.uniform(0.0, 1.0, (B, gx * gy, C))
    raw = raw.astype(np.float32)
    target = rng.uniform(0.0, 1.0, (B, H, W, C)).astype(np.float32)

    rt = torch.from_numpy(raw).to(dev).requires_grad_(True)
    img = splat.render(splat.activate(rt, gx, gy, H, W), H, W, radius=3.0)
    loss = splat.L1SSIMLoss.apply(img, torch.from_numpy(target).to(dev), 0.2)
    loss.backward()
    got = rt.grad.cpu().numpy()

    p = oa.activate(raw, gx, gy, H, W)
    img_ref, slack, mag, _ = orc.render(p, H, W, 3.0)
    check_close(img.detach().cpu().numpy(), img_ref, np.abs(img_ref), slack, "image")
    loss_ref, g_img = ol.l1_ssim(img_ref, target, 0.2)
    # the loss tests' bound (1e-5 of a mean below 1) plus the images'
    # difference (within 1e-5 per value; the loss is 1-Lipschitz in their mean)
    assert abs(float(loss.detach().cpu()) - loss_ref) <= 2e-5
    gp, gslack, gmag = orc.grad(p, g_img, H, W, 3.0)
    J = oa.activate_backward(raw, np.ones_like(gp), gx, gy, H, W)
    ref = gp * J
    tol = np.abs(J) * (1e-3 * gmag + gslack) + 1e-9
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (int(bad.sum()), float(np.max(np.abs(got - ref) / tol)))
    assert np.abs(ref).max() > 1e-6   # a non-trivial gradient
