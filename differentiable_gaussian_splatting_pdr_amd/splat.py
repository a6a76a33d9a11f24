"""PyTorch-facing wrapper of the HIP splatting library.

PyTorch provides device memory and the current HIP stream; all computation
runs in the library's kernels through :mod:`._lib`.  Tensors must live on a
ROCm device, be float32 and contiguous:

  params       [B, N, 5 + C]  (mu_x, mu_y, s1, s2, theta, a_0 .. a_{C-1})
  image        [B, H, W, C]
  grad_params  [B, N, 5 + C]
"""
from __future__ import annotations

import threading

import torch

from . import _lib


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_params(params: torch.Tensor):
    if not isinstance(params, torch.Tensor) or params.device.type != "cuda":
        raise ValueError("params must be a tensor on a ROCm device")
    if params.dtype != torch.float32 or params.dim() != 3 or params.shape[2] < 6:
        raise ValueError("params must be float32 [B, N, 5 + C] with C >= 1")
    if not params.is_contiguous():
        raise ValueError("params must be contiguous")
    B, N, P = params.shape
    return B, N, P - 5


class Workspace:
    """Caller-owned device workspace (binning records, tile lists)."""

    def __init__(self, device, nbytes: int = 0):
        self.device = torch.device(device)
        self.buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=self.device)

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr()

    @property
    def nbytes(self) -> int:
        return self.buf.numel()

    def ensure(self, nbytes: int):
        if nbytes > self.nbytes:
            self.buf = torch.empty(int(nbytes), dtype=torch.uint8, device=self.device)
        return self

    @staticmethod
    def bytes_for(B, N, H, W, C, max_pairs) -> int:
        return _lib.pdr_splat_workspace_bytes(B, N, H, W, C, max_pairs)


def _initial_pairs(B, N, H, W) -> int:
    # a few tiles per Gaussian; grown exactly on overflow
    t = _lib.pdr_splat_tile_size()
    ntiles = ((H + t - 1) // t) * ((W + t - 1) // t)
    return min(B * N * min(8, ntiles), 0x7FFFFFFF)


_FMT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


def forward(params: torch.Tensor, H: int, W: int, radius: float = 3.0,
            workspace: Workspace | None = None, image: torch.Tensor | None = None,
            dtype: torch.dtype = torch.float32):
    """Render; returns (image, workspace).  Synchronises once to check the
    list capacity and re-runs with an exactly sized workspace on overflow.
    dtype float16 / bfloat16 stores the image in that format (fp32 math)."""
    B, N, C = _check_params(params)
    dev = params.device
    ws = workspace or Workspace(dev)
    ws.ensure(Workspace.bytes_for(B, N, H, W, C, _initial_pairs(B, N, H, W)))
    if image is None:
        image = torch.empty((B, H, W, C), dtype=dtype, device=dev)
    if image.dtype not in _FMT or image.shape != (B, H, W, C) or not image.is_contiguous():
        raise ValueError("image must be contiguous [B, H, W, C] float32/float16/bfloat16")
    st = _stream(dev)
    for _ in range(2):
        if image.dtype == torch.float32:
            _lib.pdr_splat_forward(params.data_ptr(), image.data_ptr(), B, N, H, W, C, radius,
                                   ws.ptr, ws.nbytes, st)
        else:
            _lib.pdr_splat_forward_fmt(params.data_ptr(), image.data_ptr(), _FMT[image.dtype], B,
                                       N, H, W, C, radius, ws.ptr, ws.nbytes, st)
        rc, need = _lib.pdr_splat_check(ws.ptr, st)
        if rc == _lib.PDR_OK:
            return image, ws
        if rc != _lib.PDR_ERR_OVERFLOW:
            raise _lib.PdrError(rc, "pdr_splat_forward")
        ws.ensure(Workspace.bytes_for(B, N, H, W, C, need))
    raise _lib.PdrError(_lib.PDR_ERR_OVERFLOW, "pdr_splat_forward")


def backward(params: torch.Tensor, grad_image: torch.Tensor, H: int, W: int,
             radius: float = 3.0, workspace: Workspace | None = None,
             reuse_binning: bool = False, grad_params: torch.Tensor | None = None,
             check: bool = True, algo: int | None = None):
    """dL/dparams for dL/dimage; returns grad_params.  algo: None (the
    library default) or _lib.PDR_BWD_TILE / PDR_BWD_SPAN."""
    B, N, C = _check_params(params)
    dev = params.device
    if grad_image.shape != (B, H, W, C) or grad_image.dtype not in _FMT:
        raise ValueError("grad_image must be [B, H, W, C] float32/float16/bfloat16")
    grad_image = grad_image.contiguous()
    if grad_params is None:
        grad_params = torch.empty_like(params)
    st = _stream(dev)
    if workspace is None:
        reuse_binning = False
        workspace = Workspace(dev, Workspace.bytes_for(B, N, H, W, C, _initial_pairs(B, N, H, W)))
    for _ in range(2):
        if algo is not None:
            _lib.pdr_splat_backward_algo(params.data_ptr(), grad_image.data_ptr(),
                                         _FMT[grad_image.dtype], grad_params.data_ptr(), B, N, H,
                                         W, C, radius, workspace.ptr, workspace.nbytes,
                                         int(reuse_binning), algo, st)
        elif grad_image.dtype == torch.float32:
            _lib.pdr_splat_backward(params.data_ptr(), grad_image.data_ptr(),
                                    grad_params.data_ptr(), B, N, H, W, C, radius, workspace.ptr,
                                    workspace.nbytes, int(reuse_binning), st)
        else:
            _lib.pdr_splat_backward_fmt(params.data_ptr(), grad_image.data_ptr(),
                                        _FMT[grad_image.dtype], grad_params.data_ptr(), B, N, H,
                                        W, C, radius, workspace.ptr, workspace.nbytes,
                                        int(reuse_binning), st)
        if not check:
            return grad_params
        rc, need = _lib.pdr_splat_check(workspace.ptr, st)
        if rc == _lib.PDR_OK:
            return grad_params
        if rc not in (_lib.PDR_ERR_OVERFLOW, _lib.PDR_ERR_STALE):
            raise _lib.PdrError(rc, "pdr_splat_backward")
        if rc == _lib.PDR_ERR_OVERFLOW:
            workspace.ensure(Workspace.bytes_for(B, N, H, W, C, need))
        reuse_binning = False
    raise _lib.PdrError(rc, "pdr_splat_backward")


def count_support(params: torch.Tensor, H: int, W: int, radius: float = 3.0,
                  workspace: Workspace | None = None) -> int:
    """(Gaussian, pixel) pairs inside the truncation, counted on the device
    over the forward raster's traversal (the work of a forward)."""
    B, N, C = _check_params(params)
    dev = params.device
    ws = workspace or Workspace(dev)
    ws.ensure(Workspace.bytes_for(B, N, H, W, C, _initial_pairs(B, N, H, W)))
    out = torch.empty(1, dtype=torch.int64, device=dev)
    st = _stream(dev)
    for _ in range(2):
        _lib.pdr_splat_count_support(params.data_ptr(), B, N, H, W, C, radius, out.data_ptr(),
                                     ws.ptr, ws.nbytes, st)
        rc, need = _lib.pdr_splat_check(ws.ptr, st)
        if rc == _lib.PDR_OK:
            return int(out.item())
        if rc != _lib.PDR_ERR_OVERFLOW:
            raise _lib.PdrError(rc, "pdr_splat_count_support")
        ws.ensure(Workspace.bytes_for(B, N, H, W, C, need))
    raise _lib.PdrError(_lib.PDR_ERR_OVERFLOW, "pdr_splat_count_support")


def bin_lists(params: torch.Tensor, H: int, W: int, radius: float = 3.0):
    """Binning only: returns (tile_off int32 [B*nT+1], tile_list int32 [pairs])."""
    B, N, C = _check_params(params)
    dev = params.device
    t = _lib.pdr_splat_tile_size()
    nT = ((H + t - 1) // t) * ((W + t - 1) // t)
    cap = _initial_pairs(B, N, H, W)
    ws = Workspace(dev)
    st = _stream(dev)
    for _ in range(2):
        # room for per-row lists too (two-level binning runs faster with them)
        ws.ensure(Workspace.bytes_for(B, N, H, W, C, cap))
        off = torch.empty(B * nT + 1, dtype=torch.int32, device=dev)
        lst = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        _lib.pdr_splat_bin(params.data_ptr(), B, N, H, W, C, radius, off.data_ptr(),
                           lst.data_ptr(), cap, ws.ptr, ws.nbytes, st)
        rc, need = _lib.pdr_splat_check(ws.ptr, st)
        if rc == _lib.PDR_OK:
            return off, lst[:need]
        if rc != _lib.PDR_ERR_OVERFLOW:
            raise _lib.PdrError(rc, "pdr_splat_bin")
        cap = need
    raise _lib.PdrError(_lib.PDR_ERR_OVERFLOW, "pdr_splat_bin")


# ----------------------------------------------------- persistent workspaces

class _Entry:
    """One persistent workspace: its buffer, pair capacity, the call whose
    binning it holds, and the status reports still in flight."""

    def __init__(self, ws: Workspace, cap: int, key):
        self.ws = ws
        self.cap = cap
        self.key = key        # (B, N, H, W, C)
        self.gen = 0          # ids handed to calls that bin into this workspace
        self.holder = None    # id of the call whose binning the workspace holds
        self.pending = []     # (host int64[2], event, call id), oldest first
        self.free = []        # pinned int64[2] host buffers for reuse
        self.dev_status = torch.empty(2, dtype=torch.int64, device=ws.device)


class Renderer:
    """Persistent, size-keyed workspaces for repeated renders.

    A training loop renders problems of the same sizes every step; the
    one-shot :func:`forward` synchronises after each call to check the list
    capacity.  A Renderer instead keeps one workspace per (device, stream, B,
    N, H, W, C) and synchronises (pdr_splat_check) only when it creates or
    grows a workspace: the first call of a size binds with a checked forward
    and sizes the workspace to `headroom` times the pairs it needed.  Later
    calls enqueue a status report (pdr_splat_status_async, copied to pinned
    host memory) and read it once the GPU has passed it, without waiting.  A
    report of overflow -- the Gaussians grew past the headroom -- means that
    call's outputs were NaN: the workspace grows to fit and the next call on
    the Renderer that sees the report (or :meth:`flush`) raises
    :class:`_lib.PdrError` with PDR_ERR_OVERFLOW, so the loop can repeat the
    step.

    The backward of a render reuses the forward's binning when the workspace
    still holds it, and bins again otherwise (another render of the same
    sizes came in between).  Calls that share one Renderer on one stream are
    ordered; a Renderer is safe to use from several threads (autograd runs
    backward on its own thread).  At most `max_entries` sizes are kept (least
    recently used first out); `max_pending` status reports may be in flight
    per workspace before the oldest is waited for.
    """

    def __init__(self, headroom: float = 1.25, max_entries: int = 8, max_pending: int = 64):
        if not headroom >= 1.0:
            raise ValueError("headroom must be >= 1")
        self.headroom = float(headroom)
        self.max_entries = int(max_entries)
        self.max_pending = int(max_pending)
        self._entries = {}    # key -> _Entry, least recently used first
        self._lock = threading.RLock()
        self._overflowed = []  # (sizes, pairs needed, new capacity) not yet raised
        self._retired = []     # evicted entries with reports in flight

    # -- status reports
    def _track(self, e: _Entry, gen: int, st: int):
        _lib.pdr_splat_status_async(e.ws.ptr, e.dev_status.data_ptr(), st)
        if len(e.pending) >= self.max_pending:
            self._read(e, e.pending[0], wait=True)
        host = e.free.pop() if e.free else torch.empty(2, dtype=torch.int64, pin_memory=True)
        host.copy_(e.dev_status, non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(torch.cuda.current_stream(e.ws.device))
        e.pending.append((host, ev, gen))

    def _read(self, e: _Entry, item, wait: bool) -> bool:
        host, ev, gen = item
        if wait:
            ev.synchronize()
        elif not ev.query():
            return False
        e.pending.remove(item)
        rc, need = int(host[0]), int(host[1])
        e.free.append(host)
        if rc == _lib.PDR_ERR_OVERFLOW:
            self._grow(e, need)
            self._overflowed.append((e.key, need, e.cap))
        elif rc != _lib.PDR_OK:
            raise _lib.PdrError(rc, "Renderer")
        return True

    def _drain(self, e: _Entry | None, wait: bool = False):
        for x in ([e] if e is not None else []) + self._retired:
            for item in list(x.pending):
                if not self._read(x, item, wait):
                    break   # reports complete in stream order
        self._retired = [x for x in self._retired if x.pending]
        if self._overflowed:
            (B, N, H, W, C), need, cap = self._overflowed.pop(0)
            raise _lib.PdrError(
                _lib.PDR_ERR_OVERFLOW,
                "render of %d x %d Gaussians on %dx%dx%d frames needed %d (tile, Gaussian) pairs; "
                "that call's outputs are NaN and the workspace now holds %d pairs, repeat the step"
                % (B, N, H, W, C, need, cap))

    def _grow(self, e: _Entry, need: int):
        B, N, H, W, C = e.key
        cap = min(max(int(need * self.headroom) + 1024, e.cap), 0x7FFFFFFF)
        if cap > e.cap:
            e.ws.buf = torch.empty(Workspace.bytes_for(B, N, H, W, C, cap), dtype=torch.uint8,
                                   device=e.ws.device)
            e.cap = cap
            e.holder = None      # a fresh buffer holds no binning
            e.dev_status = torch.empty(2, dtype=torch.int64, device=e.ws.device)

    def flush(self):
        """Wait for every status report in flight; raises as a later call
        would if one of them overflowed."""
        with self._lock:
            for e in list(self._entries.values()):
                self._drain(e, wait=True)
            self._drain(None, wait=True)

    # -- workspaces
    def _entry(self, params, H, W, radius, launch):
        """The workspace for this problem, running `launch(ws)` in it: checked
        when the workspace is new, else with a status report.  Returns the
        entry and the id of the call."""
        B, N, C = _check_params(params)
        dev = params.device
        st = _stream(dev)
        key = (B, N, H, W, C)
        full = (dev.index, st) + key
        e = self._entries.pop(full, None)
        if e is None:
            cap = _initial_pairs(B, N, H, W)
            ws = Workspace(dev, Workspace.bytes_for(B, N, H, W, C, cap))
            for _ in range(2):
                launch(ws)
                rc, need = _lib.pdr_splat_check(ws.ptr, st)
                if rc == _lib.PDR_OK:
                    break
                if rc != _lib.PDR_ERR_OVERFLOW:
                    raise _lib.PdrError(rc, "Renderer")
                cap = need
                ws.ensure(Workspace.bytes_for(B, N, H, W, C, cap))
            else:
                raise _lib.PdrError(_lib.PDR_ERR_OVERFLOW, "Renderer")
            e = _Entry(ws, cap, key)
            e.gen = 1
            e.holder = 1
            if need * self.headroom + 1024 > e.cap:
                self._grow(e, need)           # the binning just made is gone
        else:
            self._entries[full] = e
            self._drain(e)
            launch(e.ws)
            e.gen += 1
            e.holder = e.gen
            self._track(e, e.gen, st)
        self._entries[full] = e
        while len(self._entries) > self.max_entries:
            old = self._entries.pop(next(iter(self._entries)))
            if old.pending:
                self._retired.append(old)    # its reports are still read
        return e, e.gen

    def forward(self, params, H: int, W: int, radius: float = 3.0):
        """image [B, H, W, C] (fp32); returns (image, entry, call id)."""
        B, N, C = _check_params(params)
        image = torch.empty((B, H, W, C), dtype=torch.float32, device=params.device)

        def launch(ws):
            _lib.pdr_splat_forward(params.data_ptr(), image.data_ptr(), B, N, H, W, C, radius,
                                   ws.ptr, ws.nbytes, _stream(params.device))
        with self._lock:
            e, gen = self._entry(params, H, W, radius, launch)
        return image, e, gen

    def forward_concat(self, params, pixel, H: int, W: int, radius: float = 3.0):
        """[pixel | render(params)] [B, H, W, Cp + C]; returns (out, entry, call id)."""
        B, N, C = _check_params(params)
        if pixel.dim() != 4 or pixel.shape[:3] != (B, H, W) or pixel.dtype != torch.float32:
            raise ValueError("pixel must be float32 [B, H, W, Cp]")
        pixel = pixel.contiguous()
        Cp = pixel.shape[3]
        out = torch.empty((B, H, W, Cp + C), dtype=torch.float32, device=params.device)

        def launch(ws):
            _lib.pdr_splat_forward_concat(params.data_ptr(), pixel.data_ptr(), Cp, out.data_ptr(),
                                          B, N, H, W, C, radius, ws.ptr, ws.nbytes,
                                          _stream(params.device))
        with self._lock:
            e, gen = self._entry(params, H, W, radius, launch)
        return out, e, gen

    def _backward(self, e: _Entry, gen: int, params, launch):
        with self._lock:
            self._drain(e)
            reuse = e.holder == gen
            if not reuse:            # binning again replaces what the workspace held
                e.gen += 1
                e.holder = e.gen
            launch(e.ws, reuse)
            if not reuse:
                self._track(e, e.holder, _stream(params.device))

    def backward(self, e: _Entry, gen: int, params, grad_image, H: int, W: int,
                 radius: float = 3.0):
        """dL/dparams of the render `gen` from dL/dimage (fp32)."""
        B, N, C = _check_params(params)
        grad_image = grad_image.contiguous()
        if grad_image.shape != (B, H, W, C) or grad_image.dtype != torch.float32:
            raise ValueError("grad_image must be float32 [B, H, W, C]")
        grad_params = torch.empty_like(params)

        def launch(ws, reuse):
            _lib.pdr_splat_backward(params.data_ptr(), grad_image.data_ptr(),
                                    grad_params.data_ptr(), B, N, H, W, C, radius, ws.ptr,
                                    ws.nbytes, int(reuse), _stream(params.device))
        self._backward(e, gen, params, launch)
        return grad_params

    def backward_concat(self, e: _Entry, gen: int, params, grad_out, Cp: int, H: int, W: int,
                        radius: float = 3.0, want_pixel_grad: bool = True):
        """(dL/dparams, dL/dpixel or None) of the concat render `gen`."""
        B, N, C = _check_params(params)
        grad_out = grad_out.contiguous()
        if grad_out.shape != (B, H, W, Cp + C) or grad_out.dtype != torch.float32:
            raise ValueError("grad_out must be float32 [B, H, W, Cp + C]")
        grad_params = torch.empty_like(params)
        grad_pixel = (torch.empty((B, H, W, Cp), dtype=torch.float32, device=params.device)
                      if want_pixel_grad and Cp > 0 else None)

        def launch(ws, reuse):
            _lib.pdr_splat_backward_concat(
                params.data_ptr(), grad_out.data_ptr(), Cp, grad_params.data_ptr(),
                grad_pixel.data_ptr() if grad_pixel is not None else None, B, N, H, W, C, radius,
                ws.ptr, ws.nbytes, int(reuse), _stream(params.device))
        self._backward(e, gen, params, launch)
        return grad_params, grad_pixel


_renderer = Renderer()


def default_renderer() -> Renderer:
    """The Renderer behind :func:`render` and :func:`render_concat`."""
    return _renderer


class SplatRender(torch.autograd.Function):
    """image = render(params); backward reuses the forward's binning."""

    @staticmethod
    def forward(ctx, params, H, W, radius, renderer):
        params = params.contiguous()
        r = renderer or _renderer
        image, e, gen = r.forward(params, H, W, radius)
        ctx.save_for_backward(params)
        ctx.meta = (H, W, radius, r, e, gen)
        return image

    @staticmethod
    def backward(ctx, grad_image):
        (params,) = ctx.saved_tensors
        H, W, radius, r, e, gen = ctx.meta
        g = r.backward(e, gen, params, grad_image, H, W, radius)
        return g, None, None, None, None


def render(params: torch.Tensor, H: int, W: int, radius: float = 3.0,
           renderer: Renderer | None = None) -> torch.Tensor:
    """Differentiable render of [B, N, 5 + C] Gaussians to [B, H, W, C]
    through a Renderer's persistent workspaces (the module's by default)."""
    return SplatRender.apply(params, H, W, radius, renderer)


def l1_ssim_loss(image: torch.Tensor, target: torch.Tensor, lam: float = 0.2,
                 c1: float = 1e-4, c2: float = 9e-4):
    """(loss, dloss/dimage): the L1 + SSIM training loss of [B, H, W, C]
    float32 frames, computed by the library's kernels (loss is a 0-d fp64
    device tensor)."""
    if image.shape != target.shape or image.dim() != 4:
        raise ValueError("image and target must be [B, H, W, C] of the same shape")
    if image.dtype != torch.float32 or target.dtype != torch.float32:
        raise ValueError("image and target must be float32")
    image, target = image.contiguous(), target.contiguous()
    B, H, W, C = image.shape
    dev = image.device
    ws = torch.empty(_lib.pdr_loss_workspace_bytes(B, H, W, C), dtype=torch.uint8, device=dev)
    grad = torch.empty_like(image)
    loss = torch.empty((), dtype=torch.float64, device=dev)
    _lib.pdr_loss_l1_ssim(image.data_ptr(), target.data_ptr(), B, H, W, C, lam, c1, c2,
                          grad.data_ptr(), loss.data_ptr(), ws.data_ptr(), ws.numel(),
                          _stream(dev))
    return loss, grad


class L1SSIMLoss(torch.autograd.Function):
    """loss = (1 - lam) mean|I - T| + lam (1 - mean SSIM(I, T)); gradient to I."""

    @staticmethod
    def forward(ctx, image, target, lam=0.2):
        loss, grad = l1_ssim_loss(image, target, lam)
        ctx.save_for_backward(grad)
        return loss.to(torch.float32)

    @staticmethod
    def backward(ctx, g):
        (grad,) = ctx.saved_tensors
        return grad * g.to(grad.dtype), None, None


# --------------------------------------------------------------- concat fusion

def forward_concat(params: torch.Tensor, pixel: torch.Tensor, H: int, W: int, radius: float = 3.0,
                   workspace: Workspace | None = None):
    """[pixel | render(params)] along channels: out [B, H, W, Cp + C], written
    by the forward raster (no separate concat).  Returns (out, workspace)."""
    B, N, C = _check_params(params)
    if pixel.dim() != 4 or pixel.shape[:3] != (B, H, W) or pixel.dtype != torch.float32:
        raise ValueError("pixel must be float32 [B, H, W, Cp]")
    pixel = pixel.contiguous()
    Cp = pixel.shape[3]
    dev = params.device
    ws = workspace or Workspace(dev)
    ws.ensure(Workspace.bytes_for(B, N, H, W, C, _initial_pairs(B, N, H, W)))
    out = torch.empty((B, H, W, Cp + C), dtype=torch.float32, device=dev)
    st = _stream(dev)
    for _ in range(2):
        _lib.pdr_splat_forward_concat(params.data_ptr(), pixel.data_ptr(), Cp, out.data_ptr(), B, N,
                                      H, W, C, radius, ws.ptr, ws.nbytes, st)
        rc, need = _lib.pdr_splat_check(ws.ptr, st)
        if rc == _lib.PDR_OK:
            return out, ws
        if rc != _lib.PDR_ERR_OVERFLOW:
            raise _lib.PdrError(rc, "pdr_splat_forward_concat")
        ws.ensure(Workspace.bytes_for(B, N, H, W, C, need))
    raise _lib.PdrError(_lib.PDR_ERR_OVERFLOW, "pdr_splat_forward_concat")


def backward_concat(params: torch.Tensor, grad_out: torch.Tensor, Cp: int, H: int, W: int,
                    radius: float = 3.0, workspace: Workspace | None = None,
                    reuse_binning: bool = False, want_pixel_grad: bool = True):
    """(dL/dparams, dL/dpixel or None) from dL/dout [B, H, W, Cp + C]."""
    B, N, C = _check_params(params)
    if grad_out.shape != (B, H, W, Cp + C) or grad_out.dtype != torch.float32:
        raise ValueError("grad_out must be float32 [B, H, W, Cp + C]")
    grad_out = grad_out.contiguous()
    dev = params.device
    grad_params = torch.empty_like(params)
    grad_pixel = (torch.empty((B, H, W, Cp), dtype=torch.float32, device=dev)
                  if want_pixel_grad and Cp > 0 else None)
    st = _stream(dev)
    if workspace is None:
        reuse_binning = False
        workspace = Workspace(dev, Workspace.bytes_for(B, N, H, W, C, _initial_pairs(B, N, H, W)))
    for _ in range(2):
        _lib.pdr_splat_backward_concat(params.data_ptr(), grad_out.data_ptr(), Cp,
                                       grad_params.data_ptr(),
                                       grad_pixel.data_ptr() if grad_pixel is not None else None,
                                       B, N, H, W, C, radius, workspace.ptr, workspace.nbytes,
                                       int(reuse_binning), st)
        rc, need = _lib.pdr_splat_check(workspace.ptr, st)
        if rc == _lib.PDR_OK:
            return grad_params, grad_pixel
        if rc not in (_lib.PDR_ERR_OVERFLOW, _lib.PDR_ERR_STALE):
            raise _lib.PdrError(rc, "pdr_splat_backward_concat")
        if rc == _lib.PDR_ERR_OVERFLOW:
            workspace.ensure(Workspace.bytes_for(B, N, H, W, C, need))
        reuse_binning = False
    raise _lib.PdrError(rc, "pdr_splat_backward_concat")


class SplatRenderConcat(torch.autograd.Function):
    """out = [pixel | render(params)]; backward reuses the forward's binning."""

    @staticmethod
    def forward(ctx, params, pixel, H, W, radius, renderer):
        params = params.contiguous()
        r = renderer or _renderer
        out, e, gen = r.forward_concat(params, pixel, H, W, radius)
        ctx.save_for_backward(params)
        ctx.meta = (H, W, radius, r, e, gen, pixel.shape[3])
        return out

    @staticmethod
    def backward(ctx, grad_out):
        (params,) = ctx.saved_tensors
        H, W, radius, r, e, gen, Cp = ctx.meta
        gp, gx = r.backward_concat(e, gen, params, grad_out, Cp, H, W, radius,
                                   want_pixel_grad=ctx.needs_input_grad[1])
        return gp, gx, None, None, None, None


def render_concat(params, pixel, H: int, W: int, radius: float = 3.0,
                  renderer: Renderer | None = None):
    return SplatRenderConcat.apply(params, pixel, H, W, radius, renderer)


# ------------------------------------------------------ grid and activations

def grid_init(B: int, gx: int, gy: int, H: int, W: int, C: int, init_scale: float = 0.5,
              image: torch.Tensor | None = None, device="cuda"):
    """Raw parameters [B, gx*gy, 5 + C] that activate onto the grid centres
    (scales init_scale * cell, theta 0, amplitudes from image or 0)."""
    dev = torch.device(device) if image is None else image.device
    raw = torch.empty((B, gx * gy, 5 + C), dtype=torch.float32, device=dev)
    if image is not None:
        if image.shape != (B, H, W, C) or image.dtype != torch.float32:
            raise ValueError("image must be float32 [B, H, W, C]")
        image = image.contiguous()
    _lib.pdr_grid_init(raw.data_ptr(), B, gx, gy, H, W, C, init_scale,
                       image.data_ptr() if image is not None else None, _stream(dev))
    return raw


class GridActivation(torch.autograd.Function):
    """params = activation(raw) on a gx x gy grid over an H x W frame."""

    @staticmethod
    def forward(ctx, raw, gx, gy, H, W):
        raw = raw.contiguous()
        B, N, P = raw.shape
        if N != gx * gy or raw.dtype != torch.float32 or P < 6:
            raise ValueError("raw must be float32 [B, gx*gy, 5 + C]")
        params = torch.empty_like(raw)
        _lib.pdr_params_activate(raw.data_ptr(), params.data_ptr(), B, gx, gy, H, W, P - 5,
                                 _stream(raw.device))
        ctx.save_for_backward(raw)
        ctx.meta = (gx, gy, H, W)
        return params

    @staticmethod
    def backward(ctx, grad_params):
        (raw,) = ctx.saved_tensors
        gx, gy, H, W = ctx.meta
        g = grad_params.contiguous()
        out = torch.empty_like(raw)
        B, N, P = raw.shape
        _lib.pdr_params_activate_backward(raw.data_ptr(), g.data_ptr(), out.data_ptr(), B, gx, gy,
                                          H, W, P - 5, _stream(raw.device))
        return out, None, None, None, None


def activate(raw, gx: int, gy: int, H: int, W: int):
    return GridActivation.apply(raw, gx, gy, H, W)
