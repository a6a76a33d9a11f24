"""Streams and graph capture of the C ABI on the GPU.

* Concurrent calls on two streams with distinct workspaces (the header's
  reentrancy promise): each frame set matches the oracle and the forward
  images equal those of the same calls made alone.
* A forward + backward step (binning reused) captured into a HIP graph:
  the entry points allocate nothing, synchronise nothing and record no
  memset, so the step is capturable; the graph is replayed several times
  with new parameter values and eager work in between, and every replay is
  checked against the eager result of the same values.
"""
import os

import numpy as np
import pytest

from differentiable_gaussian_splatting_pdr_amd import workloads

from helpers import check_against_oracle, check_close

pytestmark = pytest.mark.gpu

H, W, C, N, B = 64, 72, 3, 300, 4


def _inputs(seed):
    return workloads.make_custom(B, N, H, W, C, seed=seed, s_range=(0.5, 6.0), mean_margin=4.0)


def _step(lib, pt, gt, img, gp, ws, wsb, stream):
    rc = lib.pdr_splat_forward(pt.data_ptr(), img.data_ptr(), B, N, H, W, C, 3.0, ws.data_ptr(),
                               wsb, stream)
    assert rc == 0, rc
    rc = lib.pdr_splat_backward(pt.data_ptr(), gt.data_ptr(), gp.data_ptr(), B, N, H, W, C, 3.0,
                                ws.data_ptr(), wsb, 1, stream)
    assert rc == 0, rc


def _buffers(torch, dev, cap):
    from differentiable_gaussian_splatting_pdr_amd import _lib
    wsb = _lib.pdr_splat_workspace_bytes(B, N, H, W, C, cap)
    return (torch.empty((B, H, W, C), device=dev), torch.empty((B, N, 5 + C), device=dev),
            torch.empty(wsb, dtype=torch.uint8, device=dev), wsb)


def test_two_streams_distinct_workspaces(orc):
    import torch
    from differentiable_gaussian_splatting_pdr_amd import _lib
    lib = _lib.lib()
    dev = torch.device("cuda:0")
    sets = [_inputs(41), _inputs(42)]
    cap = 400_000
    # each set alone on the current stream
    alone = []
    for p, g in sets:
        pt, gt = torch.from_numpy(p).to(dev), torch.from_numpy(g).to(dev)
        img, gp, ws, wsb = _buffers(torch, dev, cap)
        st = torch.cuda.current_stream().cuda_stream
        _step(lib, pt, gt, img, gp, ws, wsb, st)
        status, _ = _lib.pdr_splat_check(ws.data_ptr(), st)
        assert status == 0
        alone.append(img.cpu().numpy())
    # both sets interleaved on two side streams (default priority)
    streams = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
    torch.cuda.synchronize()
    bufs = []
    for (p, g), s in zip(sets, streams):
        pt, gt = torch.from_numpy(p).to(dev), torch.from_numpy(g).to(dev)
        bufs.append((pt, gt) + _buffers(torch, dev, cap))
    torch.cuda.synchronize()
    for rep in range(3):
        for (pt, gt, img, gp, ws, wsb), s in zip(bufs, streams):
            rc = lib.pdr_splat_forward(pt.data_ptr(), img.data_ptr(), B, N, H, W, C, 3.0,
                                       ws.data_ptr(), wsb, s.cuda_stream)
            assert rc == 0
        for (pt, gt, img, gp, ws, wsb), s in zip(bufs, streams):
            rc = lib.pdr_splat_backward(pt.data_ptr(), gt.data_ptr(), gp.data_ptr(), B, N, H, W, C,
                                        3.0, ws.data_ptr(), wsb, 1, s.cuda_stream)
            assert rc == 0
    torch.cuda.synchronize()
    for k, ((p, g), (pt, gt, img, gp, ws, wsb), s) in enumerate(zip(sets, bufs, streams)):
        status, _ = _lib.pdr_splat_check(ws.data_ptr(), s.cuda_stream)
        assert status == 0
        im = img.cpu().numpy()
        assert np.array_equal(im, alone[k])   # the forward is deterministic
        check_against_oracle(orc, p, g, H, W, gpu={"image": im, "grad": gp.cpu().numpy()})


def test_graph_capture_and_replay(orc):
    import torch
    from differentiable_gaussian_splatting_pdr_amd import _lib
    lib = _lib.lib()
    dev = torch.device("cuda:0")
    p0, g0 = _inputs(51)
    pt, gt = torch.from_numpy(p0).to(dev), torch.from_numpy(g0).to(dev)
    img, gp, ws, wsb = _buffers(torch, dev, 400_000)
    # eager warm-up on a side stream (capture must not start on the legacy stream)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(lib, pt, gt, img, gp, ws, wsb, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(lib, pt, gt, img, gp, ws, wsb, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    img_e, gp_e, ws_e, wsb_e = _buffers(torch, dev, 400_000)
    for seed in (52, 53, 54, 55):
        p, g = _inputs(seed)
        pt.copy_(torch.from_numpy(p))
        gt.copy_(torch.from_numpy(g))
        graph.replay()
        torch.cuda.synchronize()
        got_img, got_gp = img.cpu().numpy(), gp.cpu().numpy()
        status, _ = _lib.pdr_splat_check(ws.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert status == 0
        # eager work on the same values between replays
        st = torch.cuda.current_stream().cuda_stream
        _step(lib, pt, gt, img_e, gp_e, ws_e, wsb_e, st)
        torch.cuda.synchronize()
        assert np.array_equal(got_img, img_e.cpu().numpy())
        check_against_oracle(orc, p, g, H, W, gpu={"image": got_img, "grad": got_gp})


def test_library_loaded_before_torch(orc):
    # a process that touches the binding before importing torch: the binding
    # loads torch first, so the library shares torch's HIP runtime and its
    # launches on torch's stream work (with two runtimes they fail)
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "from differentiable_gaussian_splatting_pdr_amd import _lib, workloads\n"
        "_lib.pdr_splat_bin_variant(34, 108, 11, 92)\n"
        "import numpy as np, torch\n"
        "from differentiable_gaussian_splatting_pdr_amd import splat\n"
        "p, _ = workloads.make_custom(34, 108, 11, 92, 2, seed=1000, s_range=(0.3, 9.0), mean_margin=6.0)\n"
        "img, ws = splat.forward(torch.from_numpy(p).cuda(), 11, 92)\n"
        "np.save(sys.argv[1], img.cpu().numpy())\n")
    import tempfile
    out = os.path.join(tempfile.mkdtemp(), "image.npy")
    r = subprocess.run([sys.executable, "-c", "import sys\n" + code, out], cwd=root,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    p, _ = workloads.make_custom(34, 108, 11, 92, 2, seed=1000, s_range=(0.3, 9.0), mean_margin=6.0)
    ref, slk, _, _ = orc.render(p, 11, 92)
    check_close(np.load(out), ref, np.abs(ref), slk, "image from a process that loaded the library first")
    os.remove(out)
