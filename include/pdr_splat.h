/*
 * pdr_splat.h -- C ABI of the MI355X (gfx950) differentiable 2D anisotropic
 * Gaussian splatting layer.
 *
 * The operation ("Learning Video Dynamics with Predictive Differentiable
 * Rendering": the arXiv abstract gives each Gaussian 5 + C learnable values,
 * position, scale, rotation and C channel amplitudes, rendered by a
 * differentiable 2D Gaussian renderer with arbitrary channels; the reading
 * notes on the paper, sections "Core Idea" and "Method", state that the frame
 * is the additive accumulation of the Gaussian primitives -- no opacity, no
 * compositing, no depth order; "Key Insight" and "Limitation" name the kernel
 * support as a tuned knob):
 *
 *   params[b][n] = { mu_x, mu_y, s1, s2, theta, a[0..C-1] }
 *   p = (x + 1/2, y + 1/2),  d = p - mu,  c = cos theta, s = sin theta
 *   z1 = ( c dx + s dy) / s1,   z2 = (-s dx + c dy) / s2,   q = z1^2 + z2^2
 *   w  = exp(-q / 2) if q <= radius^2 else 0
 *   image[b][y][x][ch] = sum_n a[b][n][ch] * w[b][n](x, y)
 *
 * mu is in pixels (x right, y down), s1/s2 are per-axis standard deviations
 * in pixels, theta is the angle of axis 1 in radians, radius is the
 * truncation in units of sigma.  A Gaussian is invalid -- contributes nothing
 * and gets a zero gradient -- if any of its 5 + C values is not finite or if
 * s1 <= 0 or s2 <= 0.  The backward returns dL/dparams for a given dL/dimage
 * (the truncation indicator is not differentiated).  Arithmetic is fp32;
 * Gaussians of anisotropy above 8:1 have their thin whitened coordinate
 * evaluated with compensation (a float pair), which keeps its error relative
 * to its own size however thin the Gaussian.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers (hipMalloc / torch), fp32 or
 *    int32 (one uint64 for pdr_splat_count_support; fp16 / bf16 images for
 *    the _fmt variants), C-contiguous, owned by the caller.  The library
 *    never allocates or frees device memory; everything it needs lives in
 *    the caller's workspace (256-byte aligned).
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls
 *    enqueue work and return without synchronising, except pdr_splat_check.
 *  - Arguments are validated before anything is enqueued; a negative status
 *    is returned and nothing runs.  Launch failures return PDR_ERR_HIP.
 *  - Data-dependent failures (list capacity overflow, a stale workspace on
 *    reuse) are raised on the device into the workspace header and reported
 *    by pdr_splat_check or pdr_splat_status_async.  Every element of the
 *    outputs of such a call is NaN (image, grad_params, grad_pixel); the
 *    lists and counts of pdr_splat_bin and pdr_splat_count_support are then
 *    undefined.
 *  - Reentrant: concurrent calls need distinct workspaces.
 */
#ifndef PDR_SPLAT_H
#define PDR_SPLAT_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pdr_status {
    PDR_OK = 0,
    PDR_ERR_INVALID_ARG = -1, /* null pointer, size < 1, radius not finite or <= 0, H/W too big */
    PDR_ERR_WORKSPACE = -2,   /* workspace smaller than its fixed part or misaligned */
    PDR_ERR_HIP = -3,         /* a HIP call or kernel launch failed */
    PDR_ERR_OVERFLOW = -4,    /* more (tile, Gaussian) pairs than the workspace holds */
    PDR_ERR_STALE = -5        /* backward asked to reuse binning the workspace does not hold */
};

/* Tile edge in pixels used by binning and raster (16). */
int pdr_splat_tile_size(void);

/* Inspection: which binning variant a problem of this size takes (host
 * only, no device call).  A bit set of PDR_BIN_MEMBERS (chunks are formed
 * from the Gaussians whose pixel box meets a group's tiles, instead of
 * consecutive Gaussians), PDR_BIN_COLUMNS (tile rows cut into column
 * chunks) and PDR_BIN_TWO_LEVEL (per-tile-row member lists first); 0 is
 * consecutive chunks over bands of whole tile rows.  Every variant yields
 * the same lists.  Negative pdr_status on invalid sizes. */
enum { PDR_BIN_MEMBERS = 1, PDR_BIN_COLUMNS = 2, PDR_BIN_TWO_LEVEL = 4 };
int pdr_splat_bin_variant(int B, int N, int H, int W);

/* Inspection: how many workgroups share each tile's list in the tile
 * backward raster (host only, no device call): 1 from 8192 tiles in the
 * batch (B * ceil(W/16) * ceil(H/16)), 2 from 4096, 4 from 2048, else 8.
 * Each takes a contiguous share of the tile's entries; the results are
 * the same up to the order of the atomic additions.  Negative pdr_status
 * on invalid sizes. */
int pdr_splat_backward_splits(int B, int N, int H, int W);

/* Bytes of workspace for a problem and a (tile, Gaussian) pair capacity.
 * Returns a negative pdr_status on invalid sizes.  The fixed part covers a
 * 256-byte header, 72 bytes per Gaussian (its raster record, the
 * compensation constants of a thin one, its pixel box), 16 bytes per tile
 * and 256 KiB for ordering the tiles by list length (each region rounded up
 * to 256 bytes); every pair takes 4 more bytes.  max_pairs <= 2^31 - 1.
 * Problems with many Gaussians per frame on frames of many tile bands
 * (N >= 16384 where a frame's bands would each scan all of its boxes) bin
 * in two levels: first per tile row, then per tile from the row's list.
 * Their fixed part also holds 4 bytes per (frame, tile row, block of
 * Gaussians) and 4 per (frame, tile row + 1), and every pair takes 8
 * bytes (the row lists have the same capacity as the tile lists; a
 * Gaussian's row pairs never outnumber its tile pairs).  The figure this
 * function returns covers either case.  Row lists that do not fit (a
 * workspace sized for fewer pairs, as for counting with pdr_splat_bin) cost
 * time only: binning then scans every box per group, with the same lists
 * and pair totals. */
long long pdr_splat_workspace_bytes(int B, int N, int H, int W, int C, long long max_pairs);

/* Forward.  params [B][N][5+C] fp32 -> image [B][H][W][C] fp32 (overwritten).
 * Bins the Gaussians into the workspace (kept for a later backward with
 * reuse_binning = 1).  H <= 32767, W <= 16384, N <= 2^22, B*N*(5+C) < 2^31. */
int pdr_splat_forward(const float *params, float *image, int B, int N, int H, int W, int C,
                      float radius, void *workspace, size_t workspace_bytes, void *stream);

/* Backward.  grad_image [B][H][W][C] fp32 -> grad_params [B][N][5+C] fp32
 * (overwritten: dL/dmu_x, dL/dmu_y, dL/ds1, dL/ds2, dL/dtheta, dL/da[C]).
 * reuse_binning = 1 uses the lists of the last forward on this workspace;
 * the workspace records (B, N, H, W, C, radius, params) at binning and a
 * mismatch is flagged as PDR_ERR_STALE.  The caller must not have changed
 * the parameter values in between.  reuse_binning = 0 bins again.
 * A non-finite grad_image value (NaN, +-inf) enters exactly the gradients of
 * the Gaussians whose truncated support holds its pixel, as it would in the
 * IEEE sum of their terms; every other gradient is unaffected. */
int pdr_splat_backward(const float *params, const float *grad_image, float *grad_params, int B,
                       int N, int H, int W, int C, float radius, void *workspace,
                       size_t workspace_bytes, int reuse_binning, void *stream);

/* Binning only, for inspection: writes tile_off [B*nT + 1] (exclusive scan of
 * per-tile counts, frame-major, tiles row-major, nT = ceil(W/16)*ceil(H/16))
 * and tile_list [cap] (per tile, the ascending indices n of Gaussians whose
 * pixel bounding box meets the tile).  Device pointers.  The list part is
 * only valid when pdr_splat_check reports PDR_OK and total <= cap. */
int pdr_splat_bin(const float *params, int B, int N, int H, int W, int C, float radius,
                  int *tile_off, int *tile_list, long long cap, void *workspace,
                  size_t workspace_bytes, void *stream);

/* Work count for throughput figures: bins as pdr_splat_forward does (the
 * workspace's lists are then reusable by a backward), then walks the same
 * tile lists, unit masks and fp32 whitened distance as the forward raster
 * and writes to *count (a device pointer to one unsigned 64-bit integer,
 * overwritten) the number of (Gaussian, pixel) pairs inside the truncation,
 * i.e. the pairs the forward accumulates: q <= radius^2 in the definition
 * at the top of this header, with ties at the boundary decided in fp32 as
 * the rasters decide them.  Same
 * validation, workspace and overflow protocol as pdr_splat_forward: *count
 * is only valid when pdr_splat_check reports PDR_OK. */
int pdr_splat_count_support(const float *params, int B, int N, int H, int W, int C, float radius,
                            unsigned long long *count, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Synchronises `stream`, then reports the device-side status of the last
 * call on `workspace`: PDR_OK, PDR_ERR_OVERFLOW or PDR_ERR_STALE (or
 * PDR_ERR_HIP).  *pairs_needed (may be NULL) receives the pair total of the
 * last binning. */
int pdr_splat_check(void *workspace, void *stream, long long *pairs_needed);

/* The report of pdr_splat_check without synchronising: enqueues on `stream`
 * a one-thread kernel that writes out[0] = the pdr_status of the last call
 * on `workspace` (PDR_OK, PDR_ERR_OVERFLOW or PDR_ERR_STALE) and out[1] =
 * the pair total of its binning.  `out` (two int64, 8-byte aligned) is a
 * device pointer; the caller copies it to host memory asynchronously
 * (hipMemcpyAsync into pinned memory, then an event) and reads it once the
 * event has completed.  Lets a training loop check capacity a step late
 * instead of stalling every step.  Returns PDR_ERR_INVALID_ARG for a null or misaligned `out`,
 * PDR_ERR_WORKSPACE for a misaligned workspace; the workspace must have
 * served a call before (its header is otherwise unset). */
int pdr_splat_status_async(void *workspace, long long *out, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the forward
 * of pdr_splat_forward with the library's own scratch in place of a
 * workspace.  The scratch is a static device array of
 * pdr_splat_noalloc_scratch_bytes() = 64 MiB per GPU, held from the library's
 * load until the process ends; the call allocates nothing.  It holds the
 * fixed part of pdr_splat_workspace_bytes and as many pairs as fit: a
 * problem whose fixed part exceeds it is rejected with PDR_ERR_WORKSPACE
 * before anything runs (e.g. 384 frames x 4096 Gaussians do not fit; 160 x
 * 1024 do), and one whose (tile, Gaussian) pairs exceed what remains leaves
 * the image undefined and writes PDR_ERR_OVERFLOW to *status.  status: a
 * DEVICE pointer to one int, overwritten with PDR_OK or PDR_ERR_OVERFLOW in
 * stream order.  Every call on one GPU shares that GPU's scratch: calls that
 * overlap on one GPU (other streams, other threads) race; calls ordered on
 * one stream do not.  The scratch keeps the last call's binning, but no
 * backward can reuse it. */
int pdr_splat_forward_noalloc(const float *params, float *image, int B, int N, int H, int W, int C,
                              float radius, int *status, void *stream);
long long pdr_splat_noalloc_scratch_bytes(void);

/* Static description of a status code. */
const char *pdr_splat_status_string(int status);

/* Diagnostic per-kernel timing, off by default.  While enabled, each kernel
 * launched by the entry points above is bracketed by two hipEvents recorded on
 * the caller's stream (this adds a small host cost per launch).
 * pdr_splat_timing returns the previous state.  pdr_splat_timing_read waits
 * for the recorded events and fills total_ms[k] / launches[k] (arrays of
 * PDR_KERNEL_COUNT, may be NULL) with the accumulated milliseconds and launch
 * counts per kernel class k; reset != 0 clears the accumulators.
 * PDR_K_BIN_COUNT covers the count pass (with the per-row lists of two-level
 * binning), PDR_K_SCAN the scan of the group totals and the tile order's
 * cursors, PDR_K_BIN_WRITE the list-writing pass (which scans the per-tile
 * counts of its group). */
enum pdr_kernel_id {
    PDR_K_PREPROCESS = 0, PDR_K_BIN_COUNT = 1, PDR_K_SCAN = 2, PDR_K_BIN_WRITE = 3,
    PDR_K_FORWARD_RASTER = 4, PDR_K_ZERO = 5, PDR_K_BACKWARD_RASTER = 6, PDR_K_FINALIZE = 7,
    PDR_K_LOSS_FWD = 8, PDR_K_LOSS_BWD = 9, PDR_K_LOSS_REDUCE = 10,
    PDR_K_GRID_INIT = 11, PDR_K_ACTIVATE = 12, PDR_K_ACTIVATE_BWD = 13,
    PDR_KERNEL_COUNT = 14
};
int pdr_splat_timing(int enable);
int pdr_splat_timing_read(double *total_ms, long long *launches, int reset);
const char *pdr_splat_kernel_name(int id);

/* ------------------------------------------------------------------------ */
/* Training loss ("Learning Video Dynamics with Predictive Differentiable
 * Rendering": the arXiv abstract says the model is optimised by a combined
 * L1 and SSIM loss; the reading notes' "Method" section calls L1 + SSIM
 * necessary).  Neither page gives the weighting or the SSIM window; this is
 *
 *   loss = (1 - lambda) * mean|I - T| + lambda * (1 - mean SSIM(I, T))
 *
 * with SSIM per frame and channel over the 11x11 Gaussian window of sigma
 * 1.5 (weights summing to 1), zero padding outside the frame, stabilising
 * constants c1, c2 (0.01^2 and 0.03^2 for data in [0, 1]), means over all
 * B*H*W*C values, and d|u|/du = 0 at u = 0. */

/* Workspace bytes of pdr_loss_l1_ssim (12 bytes per value for three
 * per-pixel partial-derivative maps, plus 16 bytes per workgroup of the
 * forward pass, each part rounded up to 256); negative on invalid sizes. */
long long pdr_loss_workspace_bytes(int B, int H, int W, int C);

/* image, target [B][H][W][C] fp32 -> *loss (one fp64 value on the device)
 * and grad_image [B][H][W][C] fp32 = dloss/dimage (overwritten).  Device
 * pointers; 0 <= lambda <= 1; c1, c2 > 0; B*H*W*C < 2^31 and one frame
 * H*W*C < 2^29 values (PDR_ERR_INVALID_ARG otherwise).  Deterministic. */
int pdr_loss_l1_ssim(const float *image, const float *target, int B, int H, int W, int C,
                     float lambda, float c1, float c2, float *grad_image, double *loss,
                     void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Reduced-precision image storage (page 3 of the sources, first paragraph,
 * evaluates FP16 rendering targets for splatting).  The renderer computes
 * and accumulates in fp32 exactly as pdr_splat_forward / _backward; only
 * the image it writes, or the dL/dimage it reads, is stored as fp16 or bf16
 * (IEEE binary16 / bfloat16, round to nearest even), halving those
 * tensors' bytes.  Same layouts, errors and workspace protocol. */
typedef enum { PDR_FMT_F32 = 0, PDR_FMT_F16 = 1, PDR_FMT_BF16 = 2 } pdr_format;

/* image [B][H][W][C] of the given format (2 or 4 bytes per value). */
int pdr_splat_forward_fmt(const float *params, void *image, int image_format, int B, int N, int H,
                          int W, int C, float radius, void *workspace, size_t workspace_bytes,
                          void *stream);

/* grad_image [B][H][W][C] of the given format; grad_params fp32. */
int pdr_splat_backward_fmt(const float *params, const void *grad_image, int grad_format,
                           float *grad_params, int B, int N, int H, int W, int C, float radius,
                           void *workspace, size_t workspace_bytes, int reuse_binning,
                           void *stream);

/* ------------------------------------------------------------------------ */
/* Backward algorithms.  PDR_BWD_TILE: the tile raster (16x16 tiles, one
 * wave each, per-(tile, Gaussian) wave reduction and one atomic per sum,
 * then a finalisation pass).  PDR_BWD_SPAN: tile-free (page 3 of the
 * sources, first paragraph, pairs tile-free splat processing with subgroup
 * gradient reduction): one wave per Gaussian walks the pixel spans of its
 * truncated ellipse row by row, packed 64 pixels at a time, reduces once
 * per Gaussian and stores the finished gradient row (no atomics, no
 * zeroing, no finalisation pass); it needs only the per-Gaussian records, so
 * without reuse it runs no tile binning.  C <= 16 and H*W*C < 2^29.  PDR_BWD_AUTO: the
 * library's default (what pdr_splat_backward uses): the span walk where it
 * applies and B*N <= 16384 (small, launch-bound problems), else the tile
 * raster.  Both compute the same sums within the same tolerance. */
typedef enum { PDR_BWD_AUTO = 0, PDR_BWD_TILE = 1, PDR_BWD_SPAN = 2 } pdr_backward_algo;

/* pdr_splat_backward_fmt with an explicit algorithm; PDR_ERR_INVALID_ARG for
 * PDR_BWD_SPAN outside its limits or an unknown algorithm. */
int pdr_splat_backward_algo(const float *params, const void *grad_image, int grad_format,
                            float *grad_params, int B, int N, int H, int W, int C, float radius,
                            void *workspace, size_t workspace_bytes, int reuse_binning, int algo,
                            void *stream);

/* ------------------------------------------------------------------------ */
/* Concat fusion ("Learning Video Dynamics with Predictive Differentiable
 * Rendering", reading notes, "Core Idea" and "Relation To Prior Work": the
 * Gaussian branch's rendered frame is fused with the pixel branch's coarse
 * prediction by concatenation).  out [B][H][W][Cp + C] receives, per pixel,
 * the Cp channels of pixel [B][H][W][Cp] followed by the C rendered
 * channels, written by the forward raster itself (no separate copy or
 * concat pass).  0 <= Cp and Cp + C <= 65536 (PDR_ERR_INVALID_ARG
 * otherwise); pixel may be NULL only when Cp = 0.  Same
 * workspace, errors and overflow protocol as pdr_splat_forward. */
int pdr_splat_forward_concat(const float *params, const float *pixel, int Cp, float *out, int B,
                             int N, int H, int W, int C, float radius, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Backward of pdr_splat_forward_concat: grad_out [B][H][W][Cp + C]; the last
 * C channels of every pixel drive the renderer's backward into grad_params
 * (as pdr_splat_backward), the first Cp are copied to grad_pixel
 * [B][H][W][Cp] (skipped when grad_pixel is NULL). */
int pdr_splat_backward_concat(const float *params, const float *grad_out, int Cp,
                              float *grad_params, float *grad_pixel, int B, int N, int H, int W,
                              int C, float radius, void *workspace, size_t workspace_bytes,
                              int reuse_binning, void *stream);

/* ------------------------------------------------------------------------ */
/* Adapter-side plain ops (reading notes, "Method": the adapter regresses the
 * 5 + C parameters per Gaussian from the backbone's coarse prediction;
 * "Relation To Prior Work": grid initialisation).  The pages give no
 * formulas; these are the readings:
 *
 * Grid: N = gx * gy Gaussians per frame, n = j * gx + i (row-major), cell
 * cw = W / gx, ch = H / gy, centre ((i + 1/2) cw, (j + 1/2) ch).
 * Activation of raw adapter values r [B][N][5 + C] into renderer params:
 *   mu_x = centre_x + cw tanh(r0), mu_y = centre_y + ch tanh(r1),
 *   s1 = cw exp(r2), s2 = ch exp(r3), theta = r4, a_c = r_{5+c}.
 * All pointers are device pointers, fp32, contiguous; B*N*(5+C) < 2^31,
 * N <= 2^22, H, W <= 32767; asynchronous on stream. */

/* raw [B][N][5 + C] = (0, 0, ln s0, ln s0, 0, a): activates to Gaussians on
 * the grid centres with scales s0 * cell and theta = 0; a_c is image
 * [B][H][W][C] at the pixel holding the centre, floor((2i + 1) W / (2 gx)),
 * floor((2j + 1) H / (2 gy)), or 0 when image is NULL.  init_scale = s0 > 0. */
int pdr_grid_init(float *raw, int B, int gx, int gy, int H, int W, int C, float init_scale,
                  const float *image, void *stream);

/* params [B][N][5 + C] = activation of raw (same layout; may not alias).
 * raw and params 16-byte aligned (PDR_ERR_INVALID_ARG otherwise). */
int pdr_params_activate(const float *raw, float *params, int B, int gx, int gy, int H, int W,
                        int C, void *stream);

/* grad_raw = dL/draw from grad_params = dL/dparams (elementwise chain rule
 * of the activation; grad_raw may alias grad_params).  All three pointers
 * 16-byte aligned (PDR_ERR_INVALID_ARG otherwise). */
int pdr_params_activate_backward(const float *raw, const float *grad_params, float *grad_raw,
                                 int B, int gx, int gy, int H, int W, int C, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PDR_SPLAT_H */
