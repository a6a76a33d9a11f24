"""The tile-free (span) backward against the fp64 oracle, on the GPU, over
the same cases as the tile path: ragged shapes, radii, invalid / tiny /
huge / off-screen Gaussians, needles, the five workloads (full batch),
reduced-precision dL/dI, reuse and no reuse of the forward's records, and
the stale-workspace report.  Same tolerance (helpers)."""
import numpy as np
import pytest

from differentiable_gaussian_splatting_pdr_amd import workloads

from helpers import (check_grad, check_against_oracle, check_close, gpu_forward_backward,
                     make_needles, quantize)
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def span():
    from differentiable_gaussian_splatting_pdr_amd import _lib
    return _lib.PDR_BWD_SPAN


@pytest.mark.parametrize("case", [c for c in SMALL if c[4] <= 16], ids=lambda c: "B%dN%d_%dx%dx%d" % c[:5])
@pytest.mark.parametrize("reuse", [True, False])
def test_span_small_parity(orc, case, reuse):
    B, N, H, W, C, seed, srange, margin = case
    p, g = workloads.make_custom(B, N, H, W, C, seed, s_range=srange, mean_margin=margin)
    res = gpu_forward_backward(p, g, H, W, reuse=reuse, algo=span())
    print(case, check_against_oracle(orc, p, g, H, W, gpu=res))


@pytest.mark.parametrize("radius", [1.0, 2.0, 4.5, 12.0])
def test_span_radius_variants(orc, radius):
    p, g = workloads.make_custom(2, 80, 40, 48, 2, seed=11, s_range=(0.5, 5.0), mean_margin=6.0)
    res = gpu_forward_backward(p, g, 40, 48, radius, algo=span())
    check_against_oracle(orc, p, g, 40, 48, radius, gpu=res)


def test_span_edge_cases(orc):
    H, W, C = 34, 45, 2
    p, g = workloads.make_custom(1, 12, H, W, C, seed=12)
    p[0, 0, 2] = 0.0
    p[0, 1, 3] = -2.0
    p[0, 2, 4] = np.nan
    p[0, 3, 5] = np.inf
    p[0, 4, :5] = [10.5, 20.5, 1e-3, 2e-3, 0.3]
    p[0, 5, :5] = [22.0, 17.0, 200.0, 150.0, 1.0]
    p[0, 6, :5] = [-500.0, 30.0, 2.0, 2.0, 0.0]
    p[0, 7, :5] = [16.0, 16.0, 1.0, 1.0, 0.0]
    res = gpu_forward_backward(p, g, H, W, algo=span())
    check_against_oracle(orc, p, g, H, W, gpu=res)
    assert np.all(res["grad"][0, :4] == 0.0) and np.all(res["grad"][0, 6] == 0.0)


def test_span_tiny_and_thin_gaussians(orc):
    rng = np.random.default_rng(21)
    B, N, H, W, C = 1, 80, 70, 70, 2
    p, g = workloads.make_custom(B, N, H, W, C, seed=21)
    p[0, :, 0] = rng.integers(0, W, N) + 0.5 + rng.choice([0.0, 1e-3, -0.25], N)
    p[0, :, 1] = rng.integers(0, H, N) + 0.5 + rng.choice([0.0, 2e-3, 0.4], N)
    p[0, :60, 2] = np.exp(rng.uniform(np.log(1e-3), np.log(0.4), 60))
    p[0, :60, 3] = np.exp(rng.uniform(np.log(1e-3), np.log(0.4), 60))
    # needle-like: 200:1 anisotropy at every angle (spans of one or two pixels)
    p[0, 60:, 2] = 20.0
    p[0, 60:, 3] = 0.1
    p[0, 60:, 4] = np.linspace(0, np.pi, 20)
    res = gpu_forward_backward(p, g, H, W, algo=span())
    check_against_oracle(orc, p, g, H, W, gpu=res)


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_span_workload_full_size(orc, idx):
    # gradients on every frame (16 frames spread over the 512 x 512 batch)
    wl, p, g = workloads.make_inputs(idx)
    res = gpu_forward_backward(p, g, wl.H, wl.W, algo=span())
    frames = slice(None) if wl.B * wl.H * wl.W <= 192 * 128 * 256 else np.arange(0, wl.B, wl.B // 16)
    gr, gsl, gmag = orc.grad(p[frames], g[frames], wl.H, wl.W)
    print(wl.name, check_grad(res["grad"][frames], gr, gmag, gsl, wl.name + " span grad"))


@pytest.mark.parametrize("radius", [1.0, 3.0])
def test_span_needles(orc, radius):
    p, g, H, W = make_needles()
    res = gpu_forward_backward(p, g, H, W, radius, algo=span())
    check_against_oracle(orc, p, g, H, W, radius, gpu=res)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_span_reduced_precision_grad(orc, fmt):
    import torch
    from differentiable_gaussian_splatting_pdr_amd import splat
    wl, p, g = workloads.make_inputs(2, frames=6)
    dev = torch.device("cuda:0")
    pt = torch.from_numpy(p).to(dev)
    _, ws = splat.forward(pt, wl.H, wl.W)
    gq = quantize(g, fmt)
    dt = torch.float16 if fmt == "f16" else torch.bfloat16
    gp = splat.backward(pt, torch.from_numpy(gq).to(dev).to(dt), wl.H, wl.W, workspace=ws,
                        reuse_binning=True, algo=span()).cpu().numpy()
    gr, gsl, gmag = orc.grad(p, gq, wl.H, wl.W, 3.0)
    check_grad(gp, gr, gmag, gsl, "span grad " + fmt)


def test_span_matches_tile_backward():
    # the two algorithms agree within the gradient tolerance on a full batch
    from differentiable_gaussian_splatting_pdr_amd import _lib
    wl, p, g = workloads.make_inputs(2)
    a = gpu_forward_backward(p, g, wl.H, wl.W, algo=_lib.PDR_BWD_TILE)["grad"].astype(np.float64)
    b = gpu_forward_backward(p, g, wl.H, wl.W, algo=span())["grad"].astype(np.float64)
    scale = np.maximum(np.abs(a), np.abs(b))
    rel = np.abs(a - b) / np.maximum(scale, 1e-3)
    print("max rel diff", rel.max(), "p99.99", np.percentile(rel, 99.99))
    assert np.percentile(rel, 99.9) < 1e-3


def test_span_stale_and_rejects():
    import torch
    from differentiable_gaussian_splatting_pdr_amd import _lib, splat
    wl, p, g = workloads.make_inputs(0)
    dev = torch.device("cuda:0")
    pt = torch.from_numpy(p).to(dev)
    _, ws = splat.forward(pt, wl.H, wl.W)
    other = pt.clone()
    gp = torch.empty_like(pt)
    gt = torch.from_numpy(g).to(dev)
    st = torch.cuda.current_stream().cuda_stream
    _lib.pdr_splat_backward_algo(other.data_ptr(), gt.data_ptr(), 0, gp.data_ptr(), 1, wl.N, wl.H,
                                 wl.W, wl.C, 3.0, ws.ptr, ws.nbytes, 1, span(), st)
    assert _lib.pdr_splat_check(ws.ptr, st)[0] == _lib.PDR_ERR_STALE
    L = _lib.lib()
    assert L.pdr_splat_backward_algo(pt.data_ptr(), gt.data_ptr(), 0, gp.data_ptr(), 1, wl.N, wl.H,
                                     wl.W, 17, 3.0, ws.ptr, ws.nbytes, 0, span(), None) == -1
    assert L.pdr_splat_backward_algo(pt.data_ptr(), gt.data_ptr(), 0, gp.data_ptr(), 1, wl.N, wl.H,
                                     wl.W, wl.C, 3.0, ws.ptr, ws.nbytes, 0, 7, None) == -1


def test_span_rebin_leaves_no_reusable_binning(orc):
    # a span backward that rebins builds records but no tile lists: a later
    # tile backward that asks to reuse the workspace's binning must be told
    # it is stale (not run on the lists of an earlier forward)
    import torch
    from differentiable_gaussian_splatting_pdr_amd import _lib, splat
    wl, p, g = workloads.make_inputs(1, frames=2)
    dev = torch.device("cuda:0")
    pt = torch.from_numpy(p).to(dev)
    _, ws = splat.forward(pt, wl.H, wl.W)          # lists for these params
    gt = torch.from_numpy(g).to(dev)
    gp = torch.empty_like(pt)
    st = torch.cuda.current_stream().cuda_stream
    B = pt.shape[0]
    _lib.pdr_splat_backward_algo(pt.data_ptr(), gt.data_ptr(), 0, gp.data_ptr(), B, wl.N, wl.H,
                                 wl.W, wl.C, 3.0, ws.ptr, ws.nbytes, 0, span(), st)
    assert _lib.pdr_splat_check(ws.ptr, st)[0] == _lib.PDR_OK
    _lib.pdr_splat_backward_algo(pt.data_ptr(), gt.data_ptr(), 0, gp.data_ptr(), B, wl.N, wl.H,
                                 wl.W, wl.C, 3.0, ws.ptr, ws.nbytes, 1, _lib.PDR_BWD_TILE, st)
    assert _lib.pdr_splat_check(ws.ptr, st)[0] == _lib.PDR_ERR_STALE
    # a forward restores a reusable binning
    splat.forward(pt, wl.H, wl.W, workspace=ws)
    _lib.pdr_splat_backward_algo(pt.data_ptr(), gt.data_ptr(), 0, gp.data_ptr(), B, wl.N, wl.H,
                                 wl.W, wl.C, 3.0, ws.ptr, ws.nbytes, 1, _lib.PDR_BWD_TILE, st)
    assert _lib.pdr_splat_check(ws.ptr, st)[0] == _lib.PDR_OK
    gr, gsl, gmag = orc.grad(p, g, wl.H, wl.W)
    check_grad(gp.cpu().numpy(), gr, gmag, gsl, "grad after a fresh forward")


def test_auto_choice(orc):
    # the library default takes the span walk for small problems (B*N <= 16384)
    # and the tile raster beyond; the span walk is deterministic (no atomics),
    # so the small default result equals the explicit span result bit for bit
    from differentiable_gaussian_splatting_pdr_amd import _lib
    p, g = workloads.make_custom(4, 500, 48, 40, 3, seed=61, s_range=(0.5, 6.0), mean_margin=4.0)
    auto = gpu_forward_backward(p, g, 48, 40, algo=None)["grad"]
    assert np.array_equal(auto, gpu_forward_backward(p, g, 48, 40, algo=span())["grad"])
    check_against_oracle(orc, p, g, 48, 40, gpu=gpu_forward_backward(p, g, 48, 40, algo=None))
    p, g = workloads.make_custom(9, 4000, 32, 32, 1, seed=62, s_range=(0.5, 4.0), mean_margin=2.0)
    a = gpu_forward_backward(p, g, 32, 32, algo=None)["grad"]
    t = gpu_forward_backward(p, g, 32, 32, algo=_lib.PDR_BWD_TILE)["grad"]
    s = gpu_forward_backward(p, g, 32, 32, algo=span())["grad"]
    assert not np.array_equal(a, s) or np.array_equal(t, s)   # large: not the span walk
    check_against_oracle(orc, p, g, 32, 32, gpu=gpu_forward_backward(p, g, 32, 32, algo=None))


def test_span_nonfinite_grad_image(orc):
    from test_gpu_parity import check_nonfinite, nonfinite_grad_image
    p, g, H, W = nonfinite_grad_image()
    res = gpu_forward_backward(p, g, H, W, algo=span())
    print("Gaussians reached by non-finite dL/dI:", check_nonfinite(orc, p, g, H, W, res))


@pytest.mark.parametrize("R", [4, 10, 16, 100])
def test_span_anisotropy_sweep(orc, R):
    from test_gpu_parity import anisotropy_case
    p, g, H, W = anisotropy_case(R, 100 * R)
    res = gpu_forward_backward(p, g, H, W, algo=span())
    check_against_oracle(orc, p, g, H, W, gpu=res)
