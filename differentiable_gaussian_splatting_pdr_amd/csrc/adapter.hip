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
// All three are elementwise over the B*N*(5+C) values (HBM-bound),
// coalesced, with the value's (Gaussian, slot) found by multiply-shift
// division by the invariant row length; the activation and its gradient move
// four values per thread with 16-byte accesses (buffers 16-byte aligned).
#include <math.h>
#include <stdint.h>

#include "pdr_common.hpp"
#include "pdr_internal.hpp"
#include "pdr_splat.h"

namespace pdr {

namespace {

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
    // the pixel holding the centre, floor((2i + 1) W / (2 gx)): the fp64
    // quotient of these integers (< 2^40) is within 4e-12 of the exact one,
    // which is either an integer (then exact) or at least 1/(2 gx) > 1e-7
    // from the next one, so its floor is exact
    const int px = (int)floor((double)(2u * i + 1u) * (double)g.W / (2.0 * (double)g.gx.d));
    const int py = (int)floor((double)(2u * j + 1u) * (double)g.H / (2.0 * (double)g.gy));
    v = image[(((size_t)b * g.H + py) * g.W + px) * (size_t)g.C + (k - 5)];
  }
  raw[e] = v;
}

// The activation of value e = (Gaussian gi, slot k), gi = b * N + n.
__device__ __forceinline__ float act_value(float r, uint32_t n, uint32_t k, const GridArgs &g) {
  if (k >= 4) return r;
  const uint32_t j = fdiv(n, g.gx), i = n - j * g.gx.d;
  if (k == 0) return (float)(((double)i + 0.5) * g.cw + g.cw * (double)tanhf(r));
  if (k == 1) return (float)(((double)j + 0.5) * g.ch + g.ch * (double)tanhf(r));
  const float e = expf(r);
  return (float)((k == 2 ? g.cw : g.ch) * (double)e);
}

// Its derivative applied to dL/dparams gp.
__device__ __forceinline__ float act_grad(float gp, float r, uint32_t k, const GridArgs &g) {
  if (k >= 4) return gp;
  const float cell = (float)((k & 1) ? g.ch : g.cw);
  if (k < 2) {
    // d tanh / dr = sech^2 r = 1 / cosh^2 r (1 - tanh^2 r would cancel at large |r|)
    const float c = coshf(r);
    return gp * (cell / (c * c));
  }
  return gp * (cell * expf(r));
}

// Four consecutive values per thread (16-byte loads and stores); the slot
// and grid index advance with wrap-around from the first one.
__global__ __launch_bounds__(kElemThreads) void k_activate(const float *__restrict__ raw,
                                                          float *__restrict__ params,
                                                          uint32_t total, GridArgs g) {
  const uint32_t t = blockIdx.x * kElemThreads + threadIdx.x;
  const uint32_t e0 = 4u * t;
  if (e0 >= total) return;
  const uint32_t gi = fdiv(e0, g.row);
  uint32_t k = e0 - gi * g.row.d;
  uint32_t n = gi - fdiv(gi, g.nper) * g.nper.d;
  if (e0 + 4u <= total) {
    const float4 r = reinterpret_cast<const float4 *>(raw)[t];
    float v[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = act_value(v[q], n, k, g);
      if (++k == g.row.d) {
        k = 0;
        if (++n == g.nper.d) n = 0;
      }
    }
    reinterpret_cast<float4 *>(params)[t] = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    for (uint32_t e = e0; e < total; ++e) {
      params[e] = act_value(raw[e], n, k, g);
      if (++k == g.row.d) {
        k = 0;
        if (++n == g.nper.d) n = 0;
      }
    }
  }
}

// gparams and graw may be the same buffer (each value is read, then written,
// by one thread).
__global__ __launch_bounds__(kElemThreads) void k_activate_bwd(const float *__restrict__ raw,
                                                              const float *gparams, float *graw,
                                                              uint32_t total, GridArgs g) {
  const uint32_t t = blockIdx.x * kElemThreads + threadIdx.x;
  const uint32_t e0 = 4u * t;
  if (e0 >= total) return;
  uint32_t k = e0 - fdiv(e0, g.row) * g.row.d;
  if (e0 + 4u <= total) {
    const float4 gp = reinterpret_cast<const float4 *>(gparams)[t];
    const float4 r = reinterpret_cast<const float4 *>(raw)[t];
    float v[4] = {gp.x, gp.y, gp.z, gp.w};
    const float rr[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = act_grad(v[q], rr[q], k, g);
      if (++k == g.row.d) k = 0;
    }
    reinterpret_cast<float4 *>(graw)[t] = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    for (uint32_t e = e0; e < total; ++e) {
      graw[e] = act_grad(gparams[e], raw[e], k, g);
      if (++k == g.row.d) k = 0;
    }
  }
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
  const uint32_t threads = (total + 3u) / 4u;
  PDR_TIMED(PDR_K_ACTIVATE, st,
            hipLaunchKernelGGL(k_activate, dim3((threads + kElemThreads - 1) / kElemThreads),
                               dim3(kElemThreads), 0, st, raw, params, total, g));
  return hipGetLastError();
}

hipError_t launch_activate_backward(const float *raw, const float *grad_params, float *grad_raw,
                                    int B, int gx, int gy, int H, int W, int C, hipStream_t st) {
  const GridArgs g = grid_args(B, gx, gy, H, W, C);
  const uint32_t total = (uint32_t)((long long)B * gx * gy * (5 + C));
  const uint32_t threads = (total + 3u) / 4u;
  PDR_TIMED(PDR_K_ACTIVATE_BWD, st,
            hipLaunchKernelGGL(k_activate_bwd, dim3((threads + kElemThreads - 1) / kElemThreads),
                               dim3(kElemThreads), 0, st, raw, grad_params, grad_raw, total, g));
  return hipGetLastError();
}

}  // namespace pdr
