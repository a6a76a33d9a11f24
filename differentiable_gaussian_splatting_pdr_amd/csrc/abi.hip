// abi.hip -- the extern "C" entry points declared in include/pdr_splat.h:
// argument validation, workspace carve-up and kernel launches on the
// caller's stream.  No allocation happens here.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "pdr_common.hpp"
#include "pdr_internal.hpp"
#include "pdr_splat.h"

using namespace pdr;

// The allocation-free forward's scratch (see below): 64 MiB per device.
constexpr size_t kScratchBytes = 64u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

struct Dims {
  long long BN, BT;
  int nTx, nTy;
  RowPlan rp;
};

int validate_sizes(int B, int N, int H, int W, int C, Dims *d) {
  if (B < 1 || N < 1 || H < 1 || W < 1 || C < 1) return PDR_ERR_INVALID_ARG;
  if (H > kMaxHW || W > kMaxHW || N > kMaxN) return PDR_ERR_INVALID_ARG;
  if ((W + kTileW - 1) / kTileW > kMaxGroupTiles) return PDR_ERR_INVALID_ARG;  // one tile row per bin group
  long long BN = (long long)B * N;
  // int32 parameter offsets (by division: the product could exceed 64 bits)
  if (BN > 0x7fffffffLL / (5 + (long long)C)) return PDR_ERR_INVALID_ARG;
  // below 2^31 * 2^15 * 2^14 here, as B C < 2^31
  if ((long long)B * H * W * C > (1LL << 46)) return PDR_ERR_INVALID_ARG;
  d->nTx = (W + kTileW - 1) / kTileW;
  d->nTy = (H + kTileH - 1) / kTileH;
  d->BN = BN;
  d->BT = (long long)B * d->nTx * d->nTy;
  if (d->BT + 1 > 0x7fffffffLL) return PDR_ERR_INVALID_ARG;
  d->rp = row_plan(B, N, H, W);
  return PDR_OK;
}

// Channels per output pixel of the concat layout (pixel branch + rendered):
// the row stride of the image kernels is a 32-bit int.
constexpr long long kMaxOutChannels = 65536;
int validate_out(int B, int H, int W, int Cp, int C) {
  if (Cp < 0 || (long long)Cp + C > kMaxOutChannels) return PDR_ERR_INVALID_ARG;
  if ((long long)B * H * W * (Cp + (long long)C) > (1LL << 46)) return PDR_ERR_INVALID_ARG;
  return PDR_OK;
}

int validate_radius(float radius) {
  return (isfinite(radius) && radius > 0.f) ? PDR_OK : PDR_ERR_INVALID_ARG;
}

// The workspace layout implied by its size: the fixed part, then as many
// list entries as fit (4 bytes each; 8 with per-row lists, which take a
// second list of the same capacity).
int layout_for(const Dims &d, void *ws, size_t bytes, Layout *L) {
  if (!ws) return PDR_ERR_INVALID_ARG;
  if (((uintptr_t)ws & 255u) != 0) return PDR_ERR_WORKSPACE;
  Layout fixed = make_layout(d.BN, d.BT, 0, d.rp);
  if (bytes < fixed.total) return PDR_ERR_WORKSPACE;
  long long cap = (long long)((bytes - fixed.total) / (d.rp.on ? 8 : 4));
  if (cap > 0x7fffffffLL) cap = 0x7fffffffLL;
  *L = make_layout(d.BN, d.BT, cap, d.rp);
  while (d.rp.on && cap > 0 && L->rlist + (size_t)cap * 4 > bytes) {  // alignment padding
    cap = cap > 64 ? cap - 64 : 0;
    *L = make_layout(d.BN, d.BT, cap, d.rp);
  }
  L->total = bytes;
  return PDR_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PDR_OK : PDR_ERR_HIP; }

// Which backward PDR_BWD_AUTO takes where both apply: the span walk for
// small problems, where its single launch (no zeroing, no finalisation)
// wins, and the tile raster otherwise.  Measured on MI355X (backward alone,
// the tile raster sharing each tile's list among workgroups for such small
// batches): span/tile 1.02 at 256 and 1024 Gaussians, 0.79-0.96 from 4096
// to 16384 (1 to 3 channels), 1.22-1.25 at 32768 and 1.75 at 160 x 1024.
#ifndef PDR_AUTO_SPAN_MAX_GAUSSIANS
#define PDR_AUTO_SPAN_MAX_GAUSSIANS 16384
#endif
bool auto_span(int B, int N) {
  return (long long)B * N <= PDR_AUTO_SPAN_MAX_GAUSSIANS;
}

// Forward (binning + raster) into image with Cp leading pixel-branch
// channels per pixel (Cp = 0: the plain layout).
int forward_impl(const float *params, const float *pixel, int Cp, void *image, int B, int N,
                 int H, int W, int C, float radius, void *workspace, size_t workspace_bytes,
                 void *stream, int fmt = PDR_FMT_F32) {
  Dims d;
  Layout L;
  if (!params || !image) return PDR_ERR_INVALID_ARG;
  if (fmt != PDR_FMT_F32 && fmt != PDR_FMT_F16 && fmt != PDR_FMT_BF16) return PDR_ERR_INVALID_ARG;
  int rc = validate_sizes(B, N, H, W, C, &d);
  if (rc == PDR_OK) rc = validate_radius(radius);
  if (rc == PDR_OK) rc = validate_out(B, H, W, Cp, C);
  if (rc == PDR_OK) rc = layout_for(d, workspace, workspace_bytes, &L);
  if (rc != PDR_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  char *w = (char *)workspace;
  hipError_t e = launch_binning(params, B, N, H, W, C, radius, workspace, L, (int *)(w + L.tile_off),
                                (int *)(w + L.list), L.cap, true, st);
  if (e == hipSuccess)
    e = launch_forward_raster(params, image, B, N, H, W, C, radius, workspace, L, st, pixel, Cp,
                              fmt);
  return hip_status(e);
}

int backward_impl(const float *params, const void *grad_image, int Cp, float *grad_params,
                  float *grad_pixel, int B, int N, int H, int W, int C, float radius,
                  void *workspace, size_t workspace_bytes, int reuse_binning, void *stream,
                  int fmt = PDR_FMT_F32, int algo = PDR_BWD_AUTO) {
  Dims d;
  Layout L;
  if (!params || !grad_image || !grad_params) return PDR_ERR_INVALID_ARG;
  if (fmt != PDR_FMT_F32 && fmt != PDR_FMT_F16 && fmt != PDR_FMT_BF16) return PDR_ERR_INVALID_ARG;
  int rc = validate_sizes(B, N, H, W, C, &d);
  if (rc == PDR_OK) rc = validate_radius(radius);
  if (rc == PDR_OK) rc = validate_out(B, H, W, Cp, C);
  if (rc != PDR_OK) return rc;
  if (algo != PDR_BWD_AUTO && algo != PDR_BWD_TILE && algo != PDR_BWD_SPAN) return PDR_ERR_INVALID_ARG;
  const bool span_ok = Cp == 0 && span_backward_supported(H, W, C);
  if (algo == PDR_BWD_SPAN && !span_ok) return PDR_ERR_INVALID_ARG;
  rc = layout_for(d, workspace, workspace_bytes, &L);   // arguments first, then the workspace
  if (rc != PDR_OK) return rc;
  const bool span = algo == PDR_BWD_SPAN || (algo == PDR_BWD_AUTO && span_ok && auto_span(B, N));
  hipStream_t st = (hipStream_t)stream;
  char *w = (char *)workspace;
  hipError_t e = hipSuccess;
  if (span) {
    // records only, no tile lists: the workspace is not stamped as holding
    // a binning, so a later reuse of it is reported stale
    if (!reuse_binning) e = launch_preprocess(params, B, N, H, W, C, radius, workspace, L, false, st);
    if (e == hipSuccess)
      e = launch_backward_span(params, grad_image, grad_params, B, N, H, W, C, radius, workspace, L,
                               reuse_binning != 0, st, fmt);
    return hip_status(e);
  }
  if (!reuse_binning)
    e = launch_binning(params, B, N, H, W, C, radius, workspace, L, (int *)(w + L.tile_off),
                       (int *)(w + L.list), L.cap, true, st);
  if (e == hipSuccess)
    e = launch_backward(params, grad_image, grad_params, B, N, H, W, C, radius, workspace, L,
                        reuse_binning != 0, st, grad_pixel, Cp, fmt);
  return hip_status(e);
}

// Grid of gx x gy Gaussians per frame over an H x W x C frame.
int validate_grid(int B, int gx, int gy, int H, int W, int C) {
  if (B < 1 || gx < 1 || gy < 1 || H < 1 || W < 1 || C < 1) return PDR_ERR_INVALID_ARG;
  if (H > kMaxHW || W > kMaxHW) return PDR_ERR_INVALID_ARG;
  const long long N = (long long)gx * gy;
  if (N > kMaxN) return PDR_ERR_INVALID_ARG;
  if ((long long)B * N > 0x7fffffffLL / (5 + (long long)C)) return PDR_ERR_INVALID_ARG;
  return PDR_OK;
}

// ----------------------------------------------------------------------------
// The allocation-free forward: the library's own scratch, one per device.
//
// `scratch` (top of this file) is a file-scope device array.  In host code
// its name is a
// host-side stand-in, not a device address: the device address is obtained
// once per device with hipGetSymbolAddress (the device current at the
// time) and kept in scratch_ptr[device]; only that pointer is ever passed to
// a kernel.

constexpr int kScratchDevices = 64;

std::mutex scratch_mu;
void *scratch_ptr[kScratchDevices];

// The scratch's device address on the current device (nullptr on failure).
void *scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

// The overflow status of the last binning in a workspace header, as a
// pdr_status in *out (device).
__global__ void k_status_out(const WsHeader *hdr, int *out) {
  if (threadIdx.x == 0) *out = (hdr->status & kStatusOverflow) ? PDR_ERR_OVERFLOW : PDR_OK;
}

// What pdr_splat_check reports, as two integers written in stream order:
// the pdr_status of the last call and the pair total of its binning.
__global__ void k_status_pair(const WsHeader *hdr, long long *out) {
  if (threadIdx.x != 0) return;
  const int s = hdr->status;
  out[0] = (s & kStatusOverflow) ? PDR_ERR_OVERFLOW : (s & kStatusStale) ? PDR_ERR_STALE : PDR_OK;
  out[1] = hdr->total;
}

}  // namespace

extern "C" {

int pdr_splat_tile_size(void) { return kTileW; }

int pdr_splat_bin_variant(int B, int N, int H, int W) {
  Dims d;
  const int rc = validate_sizes(B, N, H, W, 1, &d);
  return rc != PDR_OK ? rc : bin_variant(B, N, H, W);
}

int pdr_splat_backward_splits(int B, int N, int H, int W) {
  Dims d;
  const int rc = validate_sizes(B, N, H, W, 1, &d);
  return rc != PDR_OK ? rc : backward_splits(d.BT);
}

long long pdr_splat_workspace_bytes(int B, int N, int H, int W, int C, long long max_pairs) {
  Dims d;
  int rc = validate_sizes(B, N, H, W, C, &d);
  if (rc != PDR_OK) return rc;
  if (max_pairs < 0 || max_pairs > 0x7fffffffLL) return PDR_ERR_INVALID_ARG;
  return (long long)make_layout(d.BN, d.BT, max_pairs, d.rp).total;
}

int pdr_splat_forward(const float *params, float *image, int B, int N, int H, int W, int C,
                      float radius, void *workspace, size_t workspace_bytes, void *stream) {
  return forward_impl(params, nullptr, 0, image, B, N, H, W, C, radius, workspace, workspace_bytes,
                      stream);
}

int pdr_splat_forward_noalloc(const float *params, float *image, int B, int N, int H, int W, int C,
                              float radius, int *status, void *stream) {
  Dims d;
  if (!params || !image || !status) return PDR_ERR_INVALID_ARG;
  int rc = validate_sizes(B, N, H, W, C, &d);
  if (rc == PDR_OK) rc = validate_radius(radius);
  if (rc != PDR_OK) return rc;
  if (make_layout(d.BN, d.BT, 0, d.rp).total > kScratchBytes) return PDR_ERR_WORKSPACE;
  void *ws = scratch_for_current_device();
  if (!ws) return PDR_ERR_HIP;
  rc = forward_impl(params, nullptr, 0, image, B, N, H, W, C, radius, ws, kScratchBytes, stream);
  if (rc != PDR_OK) return rc;
  hipLaunchKernelGGL(k_status_out, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const WsHeader *)ws, status);
  return hip_status(hipGetLastError());
}

long long pdr_splat_noalloc_scratch_bytes(void) { return (long long)kScratchBytes; }

int pdr_splat_backward(const float *params, const float *grad_image, float *grad_params, int B,
                       int N, int H, int W, int C, float radius, void *workspace,
                       size_t workspace_bytes, int reuse_binning, void *stream) {
  return backward_impl(params, grad_image, 0, grad_params, nullptr, B, N, H, W, C, radius,
                       workspace, workspace_bytes, reuse_binning, stream);
}

int pdr_splat_forward_fmt(const float *params, void *image, int image_format, int B, int N, int H,
                          int W, int C, float radius, void *workspace, size_t workspace_bytes,
                          void *stream) {
  return forward_impl(params, nullptr, 0, image, B, N, H, W, C, radius, workspace, workspace_bytes,
                      stream, image_format);
}

int pdr_splat_backward_fmt(const float *params, const void *grad_image, int grad_format,
                           float *grad_params, int B, int N, int H, int W, int C, float radius,
                           void *workspace, size_t workspace_bytes, int reuse_binning,
                           void *stream) {
  return backward_impl(params, grad_image, 0, grad_params, nullptr, B, N, H, W, C, radius,
                       workspace, workspace_bytes, reuse_binning, stream, grad_format);
}

int pdr_splat_backward_algo(const float *params, const void *grad_image, int grad_format,
                            float *grad_params, int B, int N, int H, int W, int C, float radius,
                            void *workspace, size_t workspace_bytes, int reuse_binning, int algo,
                            void *stream) {
  return backward_impl(params, grad_image, 0, grad_params, nullptr, B, N, H, W, C, radius,
                       workspace, workspace_bytes, reuse_binning, stream, grad_format, algo);
}

int pdr_splat_forward_concat(const float *params, const float *pixel, int Cp, float *out, int B,
                             int N, int H, int W, int C, float radius, void *workspace,
                             size_t workspace_bytes, void *stream) {
  if (Cp < 0 || (Cp > 0 && !pixel)) return PDR_ERR_INVALID_ARG;
  return forward_impl(params, pixel, Cp, out, B, N, H, W, C, radius, workspace, workspace_bytes,
                      stream);
}

int pdr_splat_backward_concat(const float *params, const float *grad_out, int Cp,
                              float *grad_params, float *grad_pixel, int B, int N, int H, int W,
                              int C, float radius, void *workspace, size_t workspace_bytes,
                              int reuse_binning, void *stream) {
  if (Cp < 0) return PDR_ERR_INVALID_ARG;
  return backward_impl(params, grad_out, Cp, grad_params, grad_pixel, B, N, H, W, C, radius,
                       workspace, workspace_bytes, reuse_binning, stream);
}

int pdr_grid_init(float *raw, int B, int gx, int gy, int H, int W, int C, float init_scale,
                  const float *image, void *stream) {
  if (!raw) return PDR_ERR_INVALID_ARG;
  int rc = validate_grid(B, gx, gy, H, W, C);
  if (rc != PDR_OK) return rc;
  if (!(init_scale > 0.f) || !isfinite(init_scale)) return PDR_ERR_INVALID_ARG;
  return hip_status(launch_grid_init(raw, B, gx, gy, H, W, C, init_scale, image,
                                     (hipStream_t)stream));
}

int pdr_params_activate(const float *raw, float *params, int B, int gx, int gy, int H, int W,
                        int C, void *stream) {
  if (!raw || !params) return PDR_ERR_INVALID_ARG;
  if (((uintptr_t)raw | (uintptr_t)params) & 15u) return PDR_ERR_INVALID_ARG;
  int rc = validate_grid(B, gx, gy, H, W, C);
  if (rc != PDR_OK) return rc;
  return hip_status(launch_activate(raw, params, B, gx, gy, H, W, C, (hipStream_t)stream));
}

int pdr_params_activate_backward(const float *raw, const float *grad_params, float *grad_raw,
                                 int B, int gx, int gy, int H, int W, int C, void *stream) {
  if (!raw || !grad_params || !grad_raw) return PDR_ERR_INVALID_ARG;
  if (((uintptr_t)raw | (uintptr_t)grad_params | (uintptr_t)grad_raw) & 15u)
    return PDR_ERR_INVALID_ARG;
  int rc = validate_grid(B, gx, gy, H, W, C);
  if (rc != PDR_OK) return rc;
  return hip_status(launch_activate_backward(raw, grad_params, grad_raw, B, gx, gy, H, W, C,
                                             (hipStream_t)stream));
}

int pdr_splat_bin(const float *params, int B, int N, int H, int W, int C, float radius,
                  int *tile_off, int *tile_list, long long cap, void *workspace,
                  size_t workspace_bytes, void *stream) {
  Dims d;
  Layout L;
  if (!params || !tile_off || !tile_list || cap < 0) return PDR_ERR_INVALID_ARG;
  int rc = validate_sizes(B, N, H, W, C, &d);
  if (rc == PDR_OK) rc = validate_radius(radius);
  if (rc == PDR_OK) rc = layout_for(d, workspace, workspace_bytes, &L);
  if (rc != PDR_OK) return rc;
  if (cap > 0x7fffffffLL) cap = 0x7fffffffLL;
  // the workspace's own lists are not written: the stamp is left invalid so
  // that a later backward reusing this workspace reports PDR_ERR_STALE
  hipError_t e = launch_binning(params, B, N, H, W, C, radius, workspace, L, tile_off, tile_list,
                                cap, false, (hipStream_t)stream);
  return hip_status(e);
}

int pdr_splat_count_support(const float *params, int B, int N, int H, int W, int C, float radius,
                            unsigned long long *count, void *workspace, size_t workspace_bytes,
                            void *stream) {
  Dims d;
  Layout L;
  if (!params || !count) return PDR_ERR_INVALID_ARG;
  int rc = validate_sizes(B, N, H, W, C, &d);
  if (rc == PDR_OK) rc = validate_radius(radius);
  if (rc == PDR_OK) rc = layout_for(d, workspace, workspace_bytes, &L);
  if (rc != PDR_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  char *w = (char *)workspace;
  hipError_t e = launch_binning(params, B, N, H, W, C, radius, workspace, L, (int *)(w + L.tile_off),
                                (int *)(w + L.list), L.cap, true, st);
  if (e == hipSuccess)
    e = launch_count_support(params, B, N, H, W, C, radius, workspace, L, count, st);
  return hip_status(e);
}

int pdr_splat_check(void *workspace, void *stream, long long *pairs_needed) {
  if (!workspace) return PDR_ERR_INVALID_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return PDR_ERR_HIP;
  WsHeader h;
  if (hipMemcpy(&h, workspace, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return PDR_ERR_HIP;
  if (pairs_needed) *pairs_needed = h.total;
  if (h.status & kStatusOverflow) return PDR_ERR_OVERFLOW;
  if (h.status & kStatusStale) return PDR_ERR_STALE;
  return PDR_OK;
}

int pdr_splat_status_async(void *workspace, long long *out, void *stream) {
  if (!workspace || !out || ((uintptr_t)out & 7u) != 0) return PDR_ERR_INVALID_ARG;
  if (((uintptr_t)workspace & 255u) != 0) return PDR_ERR_WORKSPACE;
  hipLaunchKernelGGL(k_status_pair, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     (const WsHeader *)workspace, out);
  return hip_status(hipGetLastError());
}

long long pdr_loss_workspace_bytes(int B, int H, int W, int C) {
  if (B < 1 || H < 1 || W < 1 || C < 1) return PDR_ERR_INVALID_ARG;
  const long long hw = (long long)H * W;   // each factor below 2^31: no overflow
  if (hw >= (1LL << 29) || hw * C >= (1LL << 29)) return PDR_ERR_INVALID_ARG;  // 32-bit frame offsets
  if ((long long)B * (hw * C) > 0x7fffffffLL) return PDR_ERR_INVALID_ARG;
  return (long long)loss_workspace_bytes(B, H, W, C);
}

int pdr_loss_l1_ssim(const float *image, const float *target, int B, int H, int W, int C,
                     float lambda, float c1, float c2, float *grad_image, double *loss,
                     void *workspace, size_t workspace_bytes, void *stream) {
  if (!image || !target || !grad_image || !loss || !workspace) return PDR_ERR_INVALID_ARG;
  long long need = pdr_loss_workspace_bytes(B, H, W, C);
  if (need < 0) return (int)need;
  if (!(lambda >= 0.f && lambda <= 1.f) || !(c1 > 0.f) || !(c2 > 0.f) || !isfinite(c1) ||
      !isfinite(c2))
    return PDR_ERR_INVALID_ARG;
  if (((uintptr_t)workspace & 255u) != 0 || workspace_bytes < (size_t)need) return PDR_ERR_WORKSPACE;
  return hip_status(launch_loss(image, target, B, H, W, C, lambda, c1, c2, grad_image, loss,
                                workspace, (hipStream_t)stream));
}

const char *pdr_splat_status_string(int status) {
  switch (status) {
    case PDR_OK: return "ok";
    case PDR_ERR_INVALID_ARG: return "invalid argument";
    case PDR_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case PDR_ERR_HIP: return "HIP runtime or launch error";
    case PDR_ERR_OVERFLOW: return "tile list capacity exceeded";
    case PDR_ERR_STALE: return "workspace does not hold the binning of these arguments";
    default: return "unknown status";
  }
}

}  // extern "C"
