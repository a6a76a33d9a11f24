// pdr_internal.hpp -- host-side launchers shared by the C-ABI translation unit.
#pragma once

#include "pdr_common.hpp"
#include "pdr_splat.h"

namespace pdr {

// Per-kernel event timing (no-ops unless pdr_splat_timing(1)).
void timing_begin(int kid, hipStream_t st);
void timing_end(int kid, hipStream_t st);

#define PDR_TIMED(kid, st, launch) \
  do {                             \
    ::pdr::timing_begin(kid, st);  \
    launch;                        \
    ::pdr::timing_end(kid, st);    \
  } while (0)

constexpr int kMaxGroupTiles = 1024;    // tiles of one binning group (static LDS bases)
constexpr long long kMaxChunk = 4096;   // Gaussians per binning chunk (bit-matrix columns)
#ifndef PDR_BIN_TARGET_GROUPS
#define PDR_BIN_TARGET_GROUPS 2048
#endif
constexpr long long kBinTargetGroups = PDR_BIN_TARGET_GROUPS;  // binning workgroups to aim for
// ... for the second level of two-level binning, whose groups are column
// chunks of one tile row: measured on one 2048x2048 frame, 98 us of binning
// at 1024 groups against 136 us at 2048 (wider chunks)
constexpr long long kBinRowTargetGroups = 1024;
constexpr long long kBinLdsBytes = 60 * 1024 - 512;  // + 4.2 KB of static arrays stays within 64 KB
#ifndef PDR_BIN_MEMBERS
#define PDR_BIN_MEMBERS -1
#endif
constexpr int kBinMembers = PDR_BIN_MEMBERS;  // chunks of band members: -1 auto, 0 never, 1 always
constexpr int kBinMemberBands = 8;            // auto: member lists from this many bands per frame
constexpr long long kBinMemberWords = 1 << 14;  // ... and this many bit words compacted per group
constexpr int kBinMinChunkTiles = 4;         // narrowest column chunk of a band
constexpr long long kBinChunkBelow = 16;      // column chunks when a batch has fewer tile rows
constexpr long long kBinChunkTarget = 256;    // ... aiming at this many groups
#ifndef PDR_BIN_ROWS
#define PDR_BIN_ROWS -1
#endif
constexpr int kBinRows = PDR_BIN_ROWS;        // two-level binning: -1 auto, 0 never, 1 always
constexpr int kBinRowsMinN = 16384;           // auto: from this many Gaussians per frame
constexpr int kBinRowBlock = 4096;            // Gaussians per block of the row pass (at most)
constexpr int kBinRowBlockMin = 256;          // ... (at least, unless the LDS holds fewer)
constexpr long long kBinRowBlocks = 1024;     // row-pass workgroups to aim for

// K1 + count + scan + list write; tile_off/list may be the workspace's own
// regions or caller buffers (inspection entry point, stamp_valid = false so
// that the workspace does not claim to hold these lists).
hipError_t launch_binning(const float *params, int B, int N, int H, int W, int C, float radius,
                          void *ws, const Layout &L, int *tile_off, int *list, long long cap,
                          bool stamp_valid, hipStream_t st);

// Whether (and how) binning builds per-row member lists first.
RowPlan row_plan(int B, int N, int H, int W);
// bit 0: member chunks, bit 1: column chunks, bit 2: two-level (row lists)
int bin_variant(int B, int N, int H, int W);

// Per-Gaussian records only (the first step of launch_binning).
hipError_t launch_preprocess(const float *params, int B, int N, int H, int W, int C, float radius,
                             void *ws, const Layout &L, bool stamp_valid, hipStream_t st);

// Tile-free backward (one wave per Gaussian over its support spans, fused
// chain rule); needs only the records.  C <= 16, H*W*C < 2^29, plain layout.
bool span_backward_supported(int H, int W, int C);
hipError_t launch_backward_span(const float *params, const void *grad_image, float *grad_params,
                                int B, int N, int H, int W, int C, float radius, void *ws,
                                const Layout &L, bool check_stamp, hipStream_t st, int fmt);

// Forward raster: image[b][y][x][c] for all channels.  With Cp > 0 the
// output has Cp + C channels per pixel: pixel[b][y][x][0..Cp) first, then the
// rendered channels (concat fusion).
// fmt: PDR_FMT_F32 / F16 / BF16 storage of image (concat needs F32).
// Pairs inside the truncation over the workspace's lists into *count (device).
hipError_t launch_count_support(const float *params, int B, int N, int H, int W, int C,
                                float radius, void *ws, const Layout &L,
                                unsigned long long *count, hipStream_t st);
hipError_t launch_forward_raster(const float *params, void *image, int B, int N, int H, int W,
                                 int C, float radius, void *ws, const Layout &L, hipStream_t st,
                                 const float *pixel = nullptr, int Cp = 0, int fmt = PDR_FMT_F32);

// Backward: zero grad_params (and verify the binning stamp when reusing),
// raster the per-Gaussian sums with one atomic per wave per Gaussian, then
// turn the sums into gradients in place.
// With Cp > 0, grad_image has Cp + C channels per pixel; the first Cp are
// copied to grad_pixel (if not null), the rest drive the renderer.
hipError_t launch_backward(const float *params, const void *grad_image, float *grad_params, int B,
                           int N, int H, int W, int C, float radius, void *ws, const Layout &L,
                           bool check_stamp, hipStream_t st, float *grad_pixel = nullptr,
                           int Cp = 0, int fmt = PDR_FMT_F32);

// L1 + SSIM loss: grad = dloss/dimage, *loss on the device.
hipError_t launch_loss(const float *img, const float *tgt, int B, int H, int W, int C, float lam,
                       float c1, float c2, float *grad, double *loss, void *ws, hipStream_t st);
size_t loss_workspace_bytes(int B, int H, int W, int C);

// Adapter-side ops: grid initialisation, activation and its gradient.
hipError_t launch_grid_init(float *raw, int B, int gx, int gy, int H, int W, int C, float s0,
                            const float *image, hipStream_t st);
hipError_t launch_activate(const float *raw, float *params, int B, int gx, int gy, int H, int W,
                           int C, hipStream_t st);
hipError_t launch_activate_backward(const float *raw, const float *grad_params, float *grad_raw,
                                    int B, int gx, int gy, int H, int W, int C, hipStream_t st);

}  // namespace pdr
