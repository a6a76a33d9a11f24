// adapter.hip -- plain adapter-side operations around the renderer: grid
// initialisation of the Gaussians and the activation that maps raw adapter
// outputs to renderer parameters, with its gradient.
//
// "Learning Video Dynamics with Predictive Differentiable Rendering": the
// reading notes (section "Method") have the PredGS adapter regress the
// 5 + C parameters per Gaussian from the backbone's coarse prediction, and
// (section "Relation To Prior Work") name grid initialisation as part of
// the design; the pages give no formulas.  Grid: N = gx * gy Gaussians per
// frame, n = j * gx + i, cell (cw, ch) = (W / gx, H / gy), centre
// ((i + 1/2) cw, (j + 1/2) ch).  Activation of raw r:
//   mu_x = centre_x + cw tanh(r0), mu_y = centre_y + ch tanh(r1),
//   s1 = cw exp(r2), s2 = ch exp(r3), theta = r4, a_c = r_{5+c}.
// Grid initialisation writes r = (0, 0, ln s0, ln s0, 0, a), a sampled from
// an optional coarse frame at the pixel holding the centre (else 0).
//
// All three are elementwise over the B*N*(5+C) values (HBM-bound): one
// thread per value, coalesced, with the value's (Gaussian, slot) found by
// multiply-shift division by the invariant row length.
#include <math.h>
#include <stdint.h>

#include "pdr_common.hpp"
#include "pdr_internal.hpp"
#include "pdr_splat.h"

namespace pdr {

namespace {

// q = n / d for 0 <= n < 2^31 by multiply and shift (round-up method of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication"): l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1,
// q = (umulhi(n, m) + n) >> l.
struct FastDiv {
  uint32_t d, m, l;
};

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  f.l = 0;
  while ((1ull << f.l) < d) ++f.l;
  f.m = (uint32_t)((((1ull << f.l) - d) << 32) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
  return (__umulhi(n, f.m) + n) >> f.l;
}

struct GridArgs {
  FastDiv row;   // 5 + C values per Gaussian
  FastDiv nper;  // N Gaussians per frame
  FastDiv gx;    // Gaussians per grid row
  int C, H, W, gy;
  double cw, ch;
};

constexpr int kElemThreads = 256;

__device__ __forceinline__ void locate(uint32_t e, const GridArgs &g, uint32_t *b, uint32_t *n,
                                       uint32_t *k) {
  const uint32_t gi = fdiv(e, g.row);
  *k = e - gi * g.row.d;
  *b = fdiv(gi, g.nper);
  *n = gi - *b * g.nper.d;
}

__global__ __launch_bounds__(kElemThreads) void k_grid_init(float *__restrict__ raw, uint32_t total,
                                                           GridArgs g, float log_s0,
                                                           const float *__restrict__ image) {
  const uint32_t e = blockIdx.x * kElemThreads + threadIdx.x;
  if (e >= total) return;
  uint32_t b, n, k;
  locate(e, g, &b, &n, &k);
  float v = 0.f;
  if (k == 2 || k == 3) {
    v = log_s0;
  } else if (k >= 5 && image) {
    const uint32_t j = fdiv(n, g.gx), i = n - j * g.gx.d;
    // the pixel holding the centre: floor((2i + 1) W / (2 gx)), exactly
    const int px = (int)(((2ull * i + 1ull) * (uint64_t)g.W) / (2ull * g.gx.d));
    const int py = (int)(((2ull * j + 1ull) * (uint64_t)g.H) / (2ull * (uint64_t)g.gy));
    v = image[(((size_t)b * g.H + py) * g.W + px) * (size_t)g.C + (k - 5)];
  }
  raw[e] = v;
}

__global__ __launch_bounds__(kElemThreads) void k_activate(const float *__restrict__ raw,
                                                          float *__restrict__ params,
                                                          uint32_t total, GridArgs g) {
  const uint32_t e = blockIdx.x * kElemThreads + threadIdx.x;
  if (e >= total) return;
  uint32_t b, n, k;
  locate(e, g, &b, &n, &k);
  const float r = raw[e];
  float v = r;
  if (k < 4) {
    const uint32_t j = fdiv(n, g.gx), i = n - j * g.gx.d;
    if (k == 0) v = (float)(((double)i + 0.5) * g.cw + g.cw * (double)tanhf(r));
    else if (k == 1) v = (float)(((double)j + 0.5) * g.ch + g.ch * (double)tanhf(r));
    else if (k == 2) v = (float)(g.cw * (double)expf(r));
    else v = (float)(g.ch * (double)expf(r));
  }
  params[e] = v;
}

// gparams and graw may be the same buffer (each value is read, then written,
// by one thread).
__global__ __launch_bounds__(kElemThreads) void k_activate_bwd(const float *__restrict__ raw,
                                                              const float *gparams, float *graw,
                                                              uint32_t total, GridArgs g) {
  const uint32_t e = blockIdx.x * kElemThreads + threadIdx.x;
  if (e >= total) return;
  const uint32_t k = e - fdiv(e, g.row) * g.row.d;
  const float gp = gparams[e];
  float v = gp;
  if (k < 4) {
    const float r = raw[e];
    if (k < 2) {
      // d tanh / dr = sech^2 r = 1 / cosh^2 r (1 - tanh^2 r would cancel at large |r|)
      const double c = (double)coshf(r);
      v = (float)((double)gp * (k == 0 ? g.cw : g.ch) / (c * c));
    } else {
      v = (float)((double)gp * (k == 2 ? g.cw : g.ch) * (double)expf(r));
    }
  }
  graw[e] = v;
}

GridArgs grid_args(int B, int gx, int gy, int H, int W, int C) {
  GridArgs g;
  g.row = make_fastdiv((uint32_t)(5 + C));
  g.nper = make_fastdiv((uint32_t)gx * (uint32_t)gy);
  g.gx = make_fastdiv((uint32_t)gx);
  g.C = C;
  g.H = H;
  g.W = W;
  g.gy = gy;
  g.cw = (double)W / gx;
  g.ch = (double)H / gy;
  (void)B;
  return g;
}

}  // namespace

hipError_t launch_grid_init(float *raw, int B, int gx, int gy, int H, int W, int C, float s0,
                            const float *image, hipStream_t st) {
  const GridArgs g = grid_args(B, gx, gy, H, W, C);
  const uint32_t total = (uint32_t)((long long)B * gx * gy * (5 + C));
  PDR_TIMED(PDR_K_GRID_INIT, st,
            hipLaunchKernelGGL(k_grid_init, dim3((total + kElemThreads - 1) / kElemThreads),
                               dim3(kElemThreads), 0, st, raw, total, g, (float)log((double)s0),
                               image));
  return hipGetLastError();
}

hipError_t launch_activate(const float *raw, float *params, int B, int gx, int gy, int H, int W,
                           int C, hipStream_t st) {
  const GridArgs g = grid_args(B, gx, gy, H, W, C);
  const uint32_t total = (uint32_t)((long long)B * gx * gy * (5 + C));
  PDR_TIMED(PDR_K_ACTIVATE, st,
            hipLaunchKernelGGL(k_activate, dim3((total + kElemThreads - 1) / kElemThreads),
                               dim3(kElemThreads), 0, st, raw, params, total, g));
  return hipGetLastError();
}

hipError_t launch_activate_backward(const float *raw, const float *grad_params, float *grad_raw,
                                    int B, int gx, int gy, int H, int W, int C, hipStream_t st) {
  const GridArgs g = grid_args(B, gx, gy, H, W, C);
  const uint32_t total = (uint32_t)((long long)B * gx * gy * (5 + C));
  PDR_TIMED(PDR_K_ACTIVATE_BWD, st,
            hipLaunchKernelGGL(k_activate_bwd, dim3((total + kElemThreads - 1) / kElemThreads),
                               dim3(kElemThreads), 0, st, raw, grad_params, grad_raw, total, g));
  return hipGetLastError();
}

}  // namespace pdr
