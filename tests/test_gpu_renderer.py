"""Persistent workspaces (splat.Renderer) and the overflow protocol without
synchronisation: pdr_splat_status_async, NaN outputs of overflowed calls,
one capacity check per workspace over a training loop."""
import numpy as np
import pytest

from differentiable_gaussian_splatting_pdr_amd import workloads
from helpers import check_grad

pytestmark = pytest.mark.gpu


def _close(a, b, what):
    """Two GPU runs of the same kernels: equal up to the order of the
    backward's atomic additions."""
    import torch
    scale = float(b.abs().max()) if b.numel() else 0.0
    torch.testing.assert_close(a, b, rtol=1e-5, atol=1e-6 * max(scale, 1e-30), msg=what)


class _CountChecks:
    def __init__(self, monkeypatch):
        from differentiable_gaussian_splatting_pdr_amd import _lib
        self.n = 0
        real = _lib.pdr_splat_check

        def counted(*a):
            self.n += 1
            return real(*a)
        monkeypatch.setattr(_lib, "pdr_splat_check", counted)
        self._undo = lambda: monkeypatch.setattr(_lib, "pdr_splat_check", real)

    def stop(self):
        self._undo()


def test_training_loop_checks_capacity_once(orc, monkeypatch):
    """Ten autograd steps with Adam: pdr_splat_check runs once (when the
    workspace is made); every step's image equals the one-shot forward's and
    its gradient the one-shot backward's; the last step matches the oracle."""
    import torch
    from differentiable_gaussian_splatting_pdr_amd import splat
    wl, p, g = workloads.make_inputs(1, frames=6)
    H, W = wl.H, wl.W
    pt = torch.from_numpy(p).cuda().requires_grad_(True)
    gt = torch.from_numpy(g).cuda()
    opt = torch.optim.Adam([pt], lr=1e-2)
    r = splat.Renderer()
    cnt = _CountChecks(monkeypatch)
    snaps = []
    for _ in range(10):
        img = splat.render(pt, H, W, 3.0, renderer=r)
        opt.zero_grad(set_to_none=True)
        (img * gt).sum().backward()
        snaps.append((pt.detach().clone(), img.detach().clone(), pt.grad.detach().clone()))
        opt.step()
    r.flush()
    cnt.stop()
    assert cnt.n == 1, "pdr_splat_check ran %d times over 10 steps" % cnt.n
    for i, (ps, im, gr) in enumerate(snaps):
        ref, ws = splat.forward(ps, H, W, 3.0)
        assert torch.equal(im, ref), "step %d image" % i
        gref = splat.backward(ps, gt, H, W, 3.0, workspace=ws, reuse_binning=True)
        _close(gr, gref, "step %d grad" % i)
    ps, im, gr = snaps[-1]
    pn = ps.cpu().numpy()
    gr_ref, gsl, gmag = orc.grad(pn, g, H, W)
    check_grad(gr.cpu().numpy(), gr_ref, gmag, gsl, "step 10 grad vs oracle")


def test_interleaved_renders_rebin_in_backward(monkeypatch):
    """Two renders of one size before one backward: the workspace holds the
    second binning, so the first backward bins again; both gradients are
    right."""
    import torch
    from differentiable_gaussian_splatting_pdr_amd import splat
    B, N, H, W, C = 3, 300, 80, 72, 2
    p1, g1 = workloads.make_custom(B, N, H, W, C, seed=11)
    p2, g2 = workloads.make_custom(B, N, H, W, C, seed=12)
    r = splat.Renderer()
    a = torch.from_numpy(p1).cuda().requires_grad_(True)
    b = torch.from_numpy(p2).cuda().requires_grad_(True)
    G1, G2 = torch.from_numpy(g1).cuda(), torch.from_numpy(g2).cuda()
    cnt = _CountChecks(monkeypatch)
    for _ in range(3):
        a.grad = b.grad = None
        i1 = splat.render(a, H, W, 3.0, renderer=r)
        i2 = splat.render(b, H, W, 3.0, renderer=r)
        ((i1 * G1).sum() + (i2 * G2).sum()).backward()
    r.flush()
    cnt.stop()
    assert cnt.n == 1
    for x, G, img in ((a, G1, i1), (b, G2, i2)):
        ref, ws = splat.forward(x.detach(), H, W, 3.0)
        assert torch.equal(img.detach(), ref)
        _close(x.grad, splat.backward(x.detach(), G, H, W, 3.0, workspace=ws,
                                      reuse_binning=True), "grad")


def test_concat_render_through_renderer(monkeypatch):
    import torch
    from differentiable_gaussian_splatting_pdr_amd import splat
    B, N, H, W, C, Cp = 2, 200, 48, 64, 3, 5
    p, g = workloads.make_custom(B, N, H, W, C, seed=21)
    rng = np.random.default_rng(22)
    x = torch.from_numpy(rng.standard_normal((B, H, W, Cp), dtype=np.float32)).cuda()
    go = torch.from_numpy(rng.standard_normal((B, H, W, Cp + C), dtype=np.float32)).cuda()
    r = splat.Renderer()
    pt = torch.from_numpy(p).cuda().requires_grad_(True)
    xt = x.clone().requires_grad_(True)
    cnt = _CountChecks(monkeypatch)
    for _ in range(4):
        pt.grad = xt.grad = None
        out = splat.render_concat(pt, xt, H, W, 3.0, renderer=r)
        (out * go).sum().backward()
    r.flush()
    cnt.stop()
    assert cnt.n == 1
    ref, ws = splat.forward_concat(pt.detach(), x, H, W, 3.0)
    assert torch.equal(out.detach(), ref)
    gp, gx = splat.backward_concat(pt.detach(), go, Cp, H, W, 3.0, workspace=ws, reuse_binning=True)
    _close(pt.grad, gp, "concat grad_params")
    assert torch.equal(xt.grad, gx)


def _big_small(B=2, N=256, H=128, W=128, C=1):
    p, g = workloads.make_custom(B, N, H, W, C, seed=31, s_range=(0.5, 1.5))
    big = p.copy()
    big[..., 2:4] = 30.0   # each box now meets most of the 64 tiles
    return p, big, g


def test_overflow_is_reported_a_call_late_and_the_workspace_grows(monkeypatch):
    import torch
    from differentiable_gaussian_splatting_pdr_amd import _lib, splat
    p, big, _ = _big_small()
    H = W = 128
    r = splat.Renderer(headroom=1.0)
    small_t = torch.from_numpy(p).cuda()
    big_t = torch.from_numpy(big).cuda()
    cnt = _CountChecks(monkeypatch)
    splat.render(small_t, H, W, 3.0, renderer=r)        # sized for few pairs
    img = splat.render(big_t, H, W, 3.0, renderer=r)    # overflows, unchecked
    torch.cuda.synchronize()
    assert bool(torch.isnan(img).all()), "an overflowed call's image must be NaN"
    with pytest.raises(_lib.PdrError) as ei:
        r.flush()
    assert ei.value.status == _lib.PDR_ERR_OVERFLOW
    r.flush()                                           # reported once
    img2 = splat.render(big_t, H, W, 3.0, renderer=r)   # grown: right
    r.flush()
    cnt.stop()
    assert cnt.n == 1
    ref, _ = splat.forward(big_t, H, W, 3.0)
    assert torch.equal(img2, ref)


def test_overflowed_and_stale_calls_write_nan(monkeypatch):
    """Through the C ABI: a workspace of one pair overflows; the image, the
    gradients (tile and span backward, concat's pixel slice) are NaN and
    pdr_splat_status_async reports what pdr_splat_check does."""
    import torch
    from differentiable_gaussian_splatting_pdr_amd import _lib, splat
    B, N, H, W, C, Cp = 2, 256, 64, 64, 3, 2
    p, g = workloads.make_custom(B, N, H, W, C, seed=41)
    pt = torch.from_numpy(p).cuda()
    gt = torch.from_numpy(g).cuda()
    st = torch.cuda.current_stream().cuda_stream
    ws = splat.Workspace("cuda:0", splat.Workspace.bytes_for(B, N, H, W, C, 1))
    img = torch.zeros((B, H, W, C), device="cuda:0")
    gp = torch.zeros_like(pt)
    stat = torch.full((2,), 7, dtype=torch.int64, device="cuda:0")
    _lib.pdr_splat_forward(pt.data_ptr(), img.data_ptr(), B, N, H, W, C, 3.0, ws.ptr, ws.nbytes, st)
    _lib.pdr_splat_status_async(ws.ptr, stat.data_ptr(), st)
    rc, need = _lib.pdr_splat_check(ws.ptr, st)
    assert rc == _lib.PDR_ERR_OVERFLOW and need > 1
    assert stat.tolist() == [_lib.PDR_ERR_OVERFLOW, need]
    assert bool(torch.isnan(img).all())
    for algo in (_lib.PDR_BWD_TILE, _lib.PDR_BWD_SPAN):
        gp.zero_()
        _lib.pdr_splat_backward_algo(pt.data_ptr(), gt.data_ptr(), _lib.PDR_FMT_F32, gp.data_ptr(),
                                     B, N, H, W, C, 3.0, ws.ptr, ws.nbytes, 1, algo, st)
        assert _lib.pdr_splat_check(ws.ptr, st)[0] == _lib.PDR_ERR_OVERFLOW
        assert bool(torch.isnan(gp).all()), "algo %d" % algo
    # concat: the pixel branch is copied, the rendered channels and every
    # gradient are NaN
    x = torch.randn((B, H, W, Cp), device="cuda:0")
    out = torch.zeros((B, H, W, Cp + C), device="cuda:0")
    _lib.pdr_splat_forward_concat(pt.data_ptr(), x.data_ptr(), Cp, out.data_ptr(), B, N, H, W, C,
                                  3.0, ws.ptr, ws.nbytes, st)
    go = torch.randn((B, H, W, Cp + C), device="cuda:0")
    gx = torch.zeros_like(x)
    gp.zero_()
    _lib.pdr_splat_backward_concat(pt.data_ptr(), go.data_ptr(), Cp, gp.data_ptr(), gx.data_ptr(),
                                   B, N, H, W, C, 3.0, ws.ptr, ws.nbytes, 1, st)
    torch.cuda.synchronize()
    assert torch.equal(out[..., :Cp], x)
    assert bool(torch.isnan(out[..., Cp:]).all())
    assert bool(torch.isnan(gp).all()) and bool(torch.isnan(gx).all())
    # a workspace that fits; then a reuse by other parameters is stale
    ws.ensure(splat.Workspace.bytes_for(B, N, H, W, C, need))
    _lib.pdr_splat_forward(pt.data_ptr(), img.data_ptr(), B, N, H, W, C, 3.0, ws.ptr, ws.nbytes, st)
    _lib.pdr_splat_status_async(ws.ptr, stat.data_ptr(), st)
    assert _lib.pdr_splat_check(ws.ptr, st) == (_lib.PDR_OK, need)
    assert stat.tolist() == [_lib.PDR_OK, need]
    assert bool(torch.isfinite(img).all())
    other = pt.clone()
    for algo in (_lib.PDR_BWD_TILE, _lib.PDR_BWD_SPAN):
        gp.zero_()
        _lib.pdr_splat_backward_algo(other.data_ptr(), gt.data_ptr(), _lib.PDR_FMT_F32,
                                     gp.data_ptr(), B, N, H, W, C, 3.0, ws.ptr, ws.nbytes, 1, algo,
                                     st)
        _lib.pdr_splat_status_async(ws.ptr, stat.data_ptr(), st)
        assert _lib.pdr_splat_check(ws.ptr, st)[0] == _lib.PDR_ERR_STALE
        assert stat[0].item() == _lib.PDR_ERR_STALE
        assert bool(torch.isnan(gp).all()), "stale, algo %d" % algo


def test_status_async_rejects_bad_pointers():
    import torch
    from differentiable_gaussian_splatting_pdr_amd import _lib, splat
    ws = splat.Workspace("cuda:0", 4096)
    stat = torch.zeros(3, dtype=torch.int64, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    for args, rc in (((None, stat.data_ptr()), _lib.PDR_ERR_INVALID_ARG),
                     ((ws.ptr, None), _lib.PDR_ERR_INVALID_ARG),
                     ((ws.ptr, stat.data_ptr() + 4), _lib.PDR_ERR_INVALID_ARG),
                     ((ws.ptr + 8, stat.data_ptr()), _lib.PDR_ERR_WORKSPACE)):
        with pytest.raises(_lib.PdrError) as ei:
            _lib.pdr_splat_status_async(args[0], args[1], st)
        assert ei.value.status == rc


def test_evicted_workspace_still_reports_its_overflow(monkeypatch):
    """A size evicted (least recently used) while its last call's report is
    in flight: the report is still read, and flush() raises its overflow."""
    import torch
    from differentiable_gaussian_splatting_pdr_amd import _lib, splat
    p, big, _ = _big_small()
    H = W = 128
    r = splat.Renderer(headroom=1.0, max_entries=2)
    small_t, big_t = torch.from_numpy(p).cuda(), torch.from_numpy(big).cuda()
    splat.render(small_t, H, W, 3.0, renderer=r)              # size A made
    splat.render(big_t, H, W, 3.0, renderer=r)                # A overflows, unchecked
    for B in (3, 4):                                          # sizes B and C: A evicted
        q, _ = workloads.make_custom(B, 64, 48, 48, 1, seed=B)
        splat.render(torch.from_numpy(q).cuda(), 48, 48, 3.0, renderer=r)
    assert len(r._entries) == 2
    with pytest.raises(_lib.PdrError) as ei:
        r.flush()
    assert ei.value.status == _lib.PDR_ERR_OVERFLOW
    r.flush()


def test_bounded_reports_in_flight(monkeypatch):
    """With at most two reports in flight, a loop of renders waits for the
    oldest instead of growing the queue, and stays exact."""
    import torch
    from differentiable_gaussian_splatting_pdr_amd import splat
    B, N, H, W, C = 2, 200, 64, 80, 3
    p, _ = workloads.make_custom(B, N, H, W, C, seed=51)
    pt = torch.from_numpy(p).cuda()
    r = splat.Renderer(max_pending=2)
    cnt = _CountChecks(monkeypatch)
    imgs = [splat.render(pt, H, W, 3.0, renderer=r) for _ in range(8)]
    e = next(iter(r._entries.values()))
    assert len(e.pending) <= 2
    r.flush()
    cnt.stop()
    assert cnt.n == 1
    ref, _ = splat.forward(pt, H, W, 3.0)
    for img in imgs:
        assert torch.equal(img, ref)


def test_renders_from_two_threads_on_their_own_streams():
    """Two host threads, each with its own stream: one workspace per
    stream, results equal to the one-shot path."""
    import threading
    import torch
    from differentiable_gaussian_splatting_pdr_amd import splat
    r = splat.Renderer()
    out, errs = {}, []
    sets = {k: workloads.make_custom(2, 150, 40, 56, 2, seed=70 + k)[0] for k in range(2)}

    def work(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                pt = torch.from_numpy(sets[k]).cuda()
                for _ in range(4):
                    img = splat.render(pt, 40, 56, 3.0, renderer=r)
                s.synchronize()
                out[k] = img
        except Exception as e:   # reported below
            errs.append(e)
    th = [threading.Thread(target=work, args=(k,)) for k in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errs, errs
    r.flush()
    assert len(r._entries) == 2   # (device, stream, sizes) keys differ by stream
    for k in range(2):
        ref, _ = splat.forward(torch.from_numpy(sets[k]).cuda(), 40, 56, 3.0)
        assert torch.equal(out[k], ref)
