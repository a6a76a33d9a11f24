"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/pdr_splat.h declares, sizes workspaces as documented
and rejects invalid arguments before touching a device."""
import math
import os
import re
import subprocess
import sys

import pytest

from differentiable_gaussian_splatting_pdr_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pdr_splat.h")

FAKE = 0x10000  # a 256-byte aligned non-null address; never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pdr_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pdr_\w+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    L = _lib.lib()
    for f in declared_functions():
        assert hasattr(L, f)


def test_tile_size_and_status_strings():
    assert _lib.pdr_splat_tile_size() in (16, 32)
    for code in (0, -1, -2, -3, -4, -5):
        assert _lib.status_string(code) != "unknown status"
    assert _lib.status_string(-99) == "unknown status"


def test_workspace_bytes_layout():
    def a(v):
        return (v + 255) // 256 * 256
    B, N, H, W, C = 384, 4096, 128, 128, 3
    t = _lib.pdr_splat_tile_size()
    bt = B * (128 // t) ** 2
    # header, records, thin-Gaussian records, boxes, tile counts, group
    # totals, tile offsets, tile order, order histogram (8 XCD ranges x 512
    # length buckets x 16 windows)
    fixed = (a(256) + a(B * N * 32) + a(B * N * 32) + a(B * N * 8) + a(bt * 4) + a(bt * 4)
             + a((bt + 1) * 4) + a(bt * 4) + 262144)
    assert _lib.pdr_splat_workspace_bytes(B, N, H, W, C, 0) == fixed
    assert _lib.pdr_splat_workspace_bytes(B, N, H, W, C, 1000) == fixed + a(4000)
    # ragged sizes round the tile grid up
    t = _lib.pdr_splat_tile_size()
    nt = ((17 + t - 1) // t) * ((65 + t - 1) // t)
    assert _lib.pdr_splat_workspace_bytes(1, 10, 17, 65, 1, 0) == (
        a(256) + a(320) + a(320) + a(80) + a(nt * 4) + a(nt * 4) + a((nt + 1) * 4) + a(nt * 4)
        + 262144)


@pytest.mark.parametrize("args", [
    (0, 10, 16, 16, 1, 0), (1, 0, 16, 16, 1, 0), (1, 10, 0, 16, 1, 0), (1, 10, 16, 0, 1, 0),
    (1, 10, 16, 16, 0, 0), (1, 10, 16, 16, 1, -1), (1, 10, 40000, 16, 1, 0),
    (1, 10, 16, 16, 1, 2 ** 31), (1 << 20, 1 << 12, 16, 16, 1, 0), (1 << 14, 1 << 14, 16, 16, 3, 0),
    (1, (1 << 22) + 1, 16, 16, 1, 0), (1, 10, 16, 16385, 1, 0), (1, 10, 32768, 16, 1, 0),
])
def test_workspace_bytes_rejects(args):
    with pytest.raises(_lib.PdrError) as e:
        _lib.pdr_splat_workspace_bytes(*args)
    assert e.value.status == _lib.PDR_ERR_INVALID_ARG


def _fwd(**kw):
    a = dict(params=FAKE, image=FAKE, B=1, N=4, H=16, W=16, C=1, radius=3.0,
             workspace=FAKE, workspace_bytes=1 << 20, stream=None)
    a.update(kw)
    return _lib.lib().pdr_splat_forward(a["params"], a["image"], a["B"], a["N"], a["H"], a["W"],
                                        a["C"], a["radius"], a["workspace"], a["workspace_bytes"],
                                        a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(params=None), -1), (dict(image=None), -1), (dict(B=0), -1), (dict(N=-3), -1),
    (dict(C=0), -1), (dict(W=40000), -1), (dict(W=16400), -1), (dict(radius=0.0), -1), (dict(radius=-1.0), -1),
    (dict(radius=math.nan), -1), (dict(radius=math.inf), -1), (dict(workspace=None), -1),
    (dict(workspace=FAKE + 4), -2), (dict(workspace_bytes=100), -2),
])
def test_forward_validates_before_launch(kw, code):
    assert _fwd(**kw) == code


def test_backward_and_bin_validate():
    L = _lib.lib()
    assert L.pdr_splat_backward(FAKE, None, FAKE, 1, 4, 16, 16, 1, 3.0, FAKE, 1 << 20, 1, None) == -1
    assert L.pdr_splat_backward(FAKE, FAKE, FAKE, 1, 4, 16, 16, 1, float("nan"), FAKE, 1 << 20, 1,
                                None) == -1
    assert L.pdr_splat_backward(FAKE, FAKE, FAKE, 1, 4, 16, 16, 1, 3.0, FAKE, 10, 0, None) == -2
    assert L.pdr_splat_bin(FAKE, 1, 4, 16, 16, 1, 3.0, FAKE, FAKE, -1, FAKE, 1 << 20, None) == -1
    assert L.pdr_splat_bin(FAKE, 1, 4, 16, 16, 1, 3.0, None, FAKE, 5, FAKE, 1 << 20, None) == -1
    assert L.pdr_splat_check(None, None, None) == -1


def test_timing_toggle_without_device():
    assert _lib.pdr_splat_timing(True) is False
    assert _lib.pdr_splat_timing(False) is True
    t = _lib.pdr_splat_timing_read(reset=True)
    assert set(t) == {"preprocess", "bin_count", "scan", "bin_write", "forward_raster",
                      "zero_verify", "backward_raster", "finalize", "loss_fwd", "loss_bwd",
                      "loss_reduce", "grid_init", "activate", "activate_bwd"}
    assert all(v == (0.0, 0) for v in t.values())


def test_loss_entry_points_validate():
    L = _lib.lib()
    a = 256 * 1024
    need = _lib.pdr_loss_workspace_bytes(2, 40, 33, 3)
    M = 2 * 40 * 33 * 3
    # three partial maps, then one (s, |x - y|) fp64 pair per workgroup
    assert need % 256 == 0 and need >= -(-3 * M * 4 // 256) * 256 + 256
    assert need <= -(-3 * M * 4 // 256) * 256 + -(-M * 16 // 256) * 256
    with pytest.raises(_lib.PdrError):
        _lib.pdr_loss_workspace_bytes(0, 4, 4, 1)
    with pytest.raises(_lib.PdrError):   # one frame of 2^29 values
        _lib.pdr_loss_workspace_bytes(1, 1 << 15, 1 << 14, 1)
    assert _lib.pdr_loss_workspace_bytes(1, 1 << 15, (1 << 14) - 1, 1) > 0
    ok = dict(img=FAKE, tgt=FAKE, B=1, H=8, W=8, C=1, lam=0.2, c1=1e-4, c2=9e-4, grad=FAKE,
              loss=FAKE, ws=FAKE, wsb=1 << 20)

    def call(**kw):
        d = dict(ok, **kw)
        return L.pdr_loss_l1_ssim(d["img"], d["tgt"], d["B"], d["H"], d["W"], d["C"], d["lam"],
                                  d["c1"], d["c2"], d["grad"], d["loss"], d["ws"], d["wsb"], None)
    assert call(img=None) == -1 and call(loss=None) == -1 and call(ws=None) == -1
    assert call(lam=-0.1) == -1 and call(lam=1.5) == -1 and call(lam=math.nan) == -1
    assert call(c1=0.0) == -1 and call(c2=-1.0) == -1 and call(c2=math.inf) == -1
    assert call(B=0) == -1 and call(C=0) == -1
    assert call(ws=FAKE + 8) == -2 and call(wsb=16) == -2


def test_adapter_entry_points_validate():
    L = _lib.lib()
    # grid_init(raw, B, gx, gy, H, W, C, s0, image, stream)
    assert L.pdr_grid_init(None, 1, 4, 4, 16, 16, 3, 0.5, None, None) == -1
    assert L.pdr_grid_init(FAKE, 0, 4, 4, 16, 16, 3, 0.5, None, None) == -1
    assert L.pdr_grid_init(FAKE, 1, 0, 4, 16, 16, 3, 0.5, None, None) == -1
    assert L.pdr_grid_init(FAKE, 1, 4, 4, 16, 16, 0, 0.5, None, None) == -1
    assert L.pdr_grid_init(FAKE, 1, 4, 4, 16, 16, 3, 0.0, None, None) == -1
    assert L.pdr_grid_init(FAKE, 1, 4, 4, 16, 16, 3, math.inf, None, None) == -1
    assert L.pdr_grid_init(FAKE, 1, 4, 4, 40000, 16, 3, 0.5, None, None) == -1
    assert L.pdr_grid_init(FAKE, 1, 1 << 12, 1 << 11, 16, 16, 3, 0.5, None, None) == -1  # N > 2^22
    assert L.pdr_grid_init(FAKE, 1 << 10, 1 << 10, 1 << 10, 16, 16, 3, 0.5, None, None) == -1
    assert L.pdr_params_activate(None, FAKE, 1, 2, 2, 8, 8, 1, None) == -1
    assert L.pdr_params_activate(FAKE, FAKE, 1, 2, -2, 8, 8, 1, None) == -1
    assert L.pdr_params_activate_backward(FAKE, None, FAKE, 1, 2, 2, 8, 8, 1, None) == -1
    assert L.pdr_params_activate_backward(FAKE, FAKE, FAKE, 1, 2, 2, 8, 0, 1, None) == -1
    assert L.pdr_params_activate(FAKE + 4, FAKE, 1, 2, 2, 8, 8, 1, None) == -1      # 16-B alignment
    assert L.pdr_params_activate_backward(FAKE, FAKE, FAKE + 8, 1, 2, 2, 8, 8, 1, None) == -1


def test_concat_entry_points_validate():
    L = _lib.lib()
    ws = FAKE
    # forward_concat(params, pixel, Cp, out, B, N, H, W, C, radius, ws, bytes, stream)
    assert L.pdr_splat_forward_concat(FAKE, None, 2, FAKE, 1, 4, 8, 8, 1, 3.0, ws, 1 << 20, None) == -1
    assert L.pdr_splat_forward_concat(FAKE, FAKE, -1, FAKE, 1, 4, 8, 8, 1, 3.0, ws, 1 << 20, None) == -1
    assert L.pdr_splat_forward_concat(FAKE, FAKE, 2, None, 1, 4, 8, 8, 1, 3.0, ws, 1 << 20, None) == -1
    assert L.pdr_splat_forward_concat(FAKE, FAKE, 2, FAKE, 1, 4, 8, 8, 1, 0.0, ws, 1 << 20, None) == -1
    assert L.pdr_splat_forward_concat(FAKE, FAKE, 2, FAKE, 1, 4, 8, 8, 1, 3.0, ws, 16, None) == -2
    # backward_concat(params, grad_out, Cp, grad_params, grad_pixel, B, N, H, W, C, radius, ...)
    assert L.pdr_splat_backward_concat(FAKE, FAKE, -3, FAKE, None, 1, 4, 8, 8, 1, 3.0, ws, 1 << 20,
                                       0, None) == -1
    assert L.pdr_splat_backward_concat(FAKE, None, 2, FAKE, None, 1, 4, 8, 8, 1, 3.0, ws, 1 << 20,
                                       0, None) == -1
    assert L.pdr_splat_backward_concat(FAKE, FAKE, 2, FAKE, None, 1, 4, 8, 8, 1, 3.0, ws + 8,
                                       1 << 20, 0, None) == -2


# The binning variant rule (host logic): bit 0 member chunks, bit 1 column
# chunks, bit 2 two-level.  Column chunks only when the whole batch has
# fewer than 16 tile rows; member chunks when a frame has at least 8 groups
# and a group would compact at least 2^19 bit words; two-level when that
# member rule holds with N >= 16384.
@pytest.mark.parametrize("shape,variant", [
    ((1, 256, 64, 64), 0), ((160, 1024, 64, 64), 0), ((384, 4096, 128, 128), 0),
    ((192, 8192, 128, 256), 0),            # the batched workloads: consecutive chunks
    ((80, 65536, 512, 512), 5),            # 2560 tile rows: a group per row, no column chunks
    ((1, 12000, 256, 1024), 1),            # 16 rows of 64 tiles: 12000 * 64 >= 2^19
    ((1, 16383, 512, 512), 0),             # 32 rows of 32 tiles: 16383 * 32 < 2^19
    ((1, 16384, 512, 512), 7),             # ... 16384 * 32 = 2^19 and N >= 16384
    ((1, 3000, 64, 1000), 2), ((1, 20000, 20, 16384), 2),
    ((1, 16000, 240, 10240), 3),           # 15 rows cut into 36-tile chunks
    ((1, 262144, 2048, 2048), 7), ((4, 65536, 1024, 1024), 7),
])
def test_bin_variant_rule(shape, variant):
    assert _lib.lib().pdr_splat_bin_variant(*shape) == variant


def test_bin_variant_validates():
    L = _lib.lib()
    assert L.pdr_splat_bin_variant(0, 10, 16, 16) == _lib.PDR_ERR_INVALID_ARG
    assert L.pdr_splat_bin_variant(1, 10, 40000, 16) == _lib.PDR_ERR_INVALID_ARG
    with pytest.raises(_lib.PdrError):
        _lib.pdr_splat_bin_variant(1, 0, 16, 16)


def test_count_support_validates():
    L = _lib.lib()
    # null count, null params, zero frames, bad radius: rejected before any launch
    assert L.pdr_splat_count_support(FAKE, 1, 4, 16, 16, 1, 3.0, None, FAKE, 1 << 20, None) == -1
    assert L.pdr_splat_count_support(None, 1, 4, 16, 16, 1, 3.0, FAKE, FAKE, 1 << 20, None) == -1
    assert L.pdr_splat_count_support(FAKE, 0, 4, 16, 16, 1, 3.0, FAKE, FAKE, 1 << 20, None) == -1
    assert L.pdr_splat_count_support(FAKE, 1, 4, 16, 16, 1, -1.0, FAKE, FAKE, 1 << 20, None) == -1
    assert L.pdr_splat_count_support(FAKE, 1, 4, 16, 16, 1, 3.0, FAKE, FAKE, 16, None) == -2


def test_binding_loads_torch_first():
    # the binding imports torch before loading the library (one HIP runtime
    # per process): checked in a fresh interpreter that touches the library
    # before anything else
    code = ("import sys; from differentiable_gaussian_splatting_pdr_amd import _lib; "
            "assert 'torch' not in sys.modules; _lib.lib(); assert 'torch' in sys.modules")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]


def test_no_fallback_without_the_library():
    """The bindings only marshal arguments: with the library missing every
    call raises, and rendering a CPU tensor raises instead of computing
    (there is no CPU path).  Run in a child process so that this process's
    loaded library is untouched."""
    code = r'''
import torch
from differentiable_gaussian_splatting_pdr_amd import _lib, splat
_lib.LIB_PATH = "/nonexistent/libpdrsplat.so"
_lib._lib = None
try:
    _lib.pdr_splat_tile_size()
except RuntimeError as e:
    assert "not built" in str(e), e
else:
    raise SystemExit("binding ran without the library")
try:
    splat.render(torch.zeros(1, 4, 8), 16, 16)
except Exception as e:
    print("render raised", type(e).__name__)
else:
    raise SystemExit("render produced an image without the library")
'''
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "render raised" in r.stdout


@pytest.mark.parametrize("B,H,W,S", [(1, 16, 16, 8), (2047, 16, 16, 8), (2048, 16, 16, 4),
                                     (4095, 16, 16, 4), (4096, 16, 16, 2), (8191, 16, 16, 2),
                                     (8192, 16, 16, 1), (1, 1024, 2048, 1), (2, 1000, 1000, 2),
                                     (40, 128, 128, 4), (72, 128, 128, 2), (130, 128, 128, 1)])
def test_backward_splits_rule(B, H, W, S):
    """Workgroups per tile of the tile backward, by the batch's tile count."""
    assert _lib.pdr_splat_backward_splits(B, 64, H, W) == S


def test_backward_splits_validates():
    for args in ((0, 64, 16, 16), (1, 0, 16, 16), (1, 64, 0, 16), (1, 64, 16, 40000)):
        with pytest.raises(_lib.PdrError):
            _lib.pdr_splat_backward_splits(*args)
