// loss.hip -- combined L1 + SSIM training loss of rendered frames and its
// gradient with respect to the rendered image.
//
//   loss = (1 - lam) mean|I - T| + lam (1 - mean SSIM(I, T))
//
// SSIM per frame and channel with the 11x11 Gaussian window (sigma 1.5,
// weights summing to 1), zero padding outside the frame, constants c1, c2;
// means over all B*H*W*C values; d|u|/du = 0 at u = 0.
//
// k_ssim_fwd: per 32x32 output tile and channel, load x = I and y = T with a
//   5-pixel halo into LDS, take the five window moments (x, y, x^2, y^2, xy)
//   with a separable pass (rows, then columns), and per pixel form
//   s = A1 A2 / (B1 B2) and the three partial derivatives of s with respect
//   to mu_x, m_xx and m_xy; write those maps, and per-workgroup sums of s and
//   |x - y| (fp64).
// k_ssim_bwd: per tile and channel, correlate the three partial maps with
//   the window (same separable scheme) and combine:
//   dL/dx = (1 - lam)/M sign(x - y)
//           - lam/M [ G*P_mu + 2 x G*P_xx + y G*P_xy ].
// k_loss_reduce: one workgroup adds the per-workgroup sums in a fixed order.
#include <math.h>
#include <stdint.h>

#include "pdr_common.hpp"
#include "pdr_internal.hpp"
#include "pdr_splat.h"

namespace pdr {

constexpr int kLT = 32;                 // output tile edge
constexpr int kLR = 5;                  // window radius (11 taps)
constexpr int kLIn = kLT + 2 * kLR;     // 42: tile with halo
constexpr int kLThreads = 256;

struct Taps {
  float g[2 * kLR + 1];
};

__device__ __forceinline__ double block_sum_d(double v, double *red) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kLThreads / kWave; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Load a (kLIn x kLIn) tile of channel c with zero padding outside the frame.
__device__ __forceinline__ void load_halo(float (*dst)[kLIn], const float *__restrict__ src, int H,
                                          int W, int C, int c, int y0, int x0) {
  for (int i = threadIdx.x; i < kLIn * kLIn; i += kLThreads) {
    const int r = i / kLIn, q = i % kLIn;
    const int yy = y0 - kLR + r, xx = x0 - kLR + q;
    dst[r][q] = (yy >= 0 && yy < H && xx >= 0 && xx < W) ? src[((size_t)yy * W + xx) * C + c] : 0.f;
  }
}

__global__ __launch_bounds__(kLThreads) void k_ssim_fwd(const float *__restrict__ img,
                                                        const float *__restrict__ tgt, int B,
                                                        int H, int W, int C, Taps tp, float c1,
                                                        float c2, float *__restrict__ pmaps,
                                                        double *__restrict__ partial) {
  __shared__ float sx[kLIn][kLIn], sy[kLIn][kLIn];
  __shared__ float hs[5][kLIn][kLT];
  __shared__ double red[kLThreads / kWave];
  const int ntx = (W + kLT - 1) / kLT, nty = (H + kLT - 1) / kLT;
  const int blk = blockIdx.x;
  const int b = blk / (ntx * nty), t = blk % (ntx * nty);
  const int x0 = (t % ntx) * kLT, y0 = (t / ntx) * kLT;
  const size_t fo = (size_t)b * H * W * C;
  const size_t M = (size_t)B * H * W * C;
  double acc_s = 0.0, acc_l1 = 0.0;
  for (int c = 0; c < C; ++c) {
    load_halo(sx, img + fo, H, W, C, c, y0, x0);
    load_halo(sy, tgt + fo, H, W, C, c, y0, x0);
    __syncthreads();
    // rows: horizontal window sums of the five quantities, for all halo rows
    for (int i = threadIdx.x; i < kLIn * kLT; i += kLThreads) {
      const int r = i / kLT, q = i % kLT;
      float a = 0.f, bb = 0.f, aa = 0.f, bbb = 0.f, ab = 0.f;
#pragma unroll
      for (int k = 0; k < 2 * kLR + 1; ++k) {
        const float xv = sx[r][q + k], yv = sy[r][q + k], g = tp.g[k];
        a += g * xv;
        bb += g * yv;
        aa += g * xv * xv;
        bbb += g * yv * yv;
        ab += g * xv * yv;
      }
      hs[0][r][q] = a;
      hs[1][r][q] = bb;
      hs[2][r][q] = aa;
      hs[3][r][q] = bbb;
      hs[4][r][q] = ab;
    }
    __syncthreads();
    // columns, then SSIM and its partials per output pixel
    for (int i = threadIdx.x; i < kLT * kLT; i += kLThreads) {
      const int r = i / kLT, q = i % kLT;
      const int yy = y0 + r, xx = x0 + q;
      float m[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 2 * kLR + 1; ++k) {
        const float g = tp.g[k];
#pragma unroll
        for (int j = 0; j < 5; ++j) m[j] += g * hs[j][r + k][q];
      }
      if (yy < H && xx < W) {
        const float mx = m[0], my = m[1];
        const float a1 = 2.f * mx * my + c1;
        const float a2 = 2.f * (m[4] - mx * my) + c2;
        const float b1 = mx * mx + my * my + c1;
        const float b2 = (m[2] - mx * mx) + (m[3] - my * my) + c2;
        const float ib1 = 1.f / b1, ib2 = 1.f / b2;
        const float s = a1 * a2 * ib1 * ib2;
        const float p_mu = 2.f * my * (a2 - a1) * ib1 * ib2 - 2.f * mx * s * (ib1 - ib2);
        const float p_xx = -s * ib2;
        const float p_xy = 2.f * a1 * ib1 * ib2;
        const size_t o = fo + ((size_t)yy * W + xx) * C + c;
        pmaps[o] = p_mu;
        pmaps[M + o] = p_xx;
        pmaps[2 * M + o] = p_xy;
        acc_s += (double)s;
        acc_l1 += (double)fabsf(sx[r + kLR][q + kLR] - sy[r + kLR][q + kLR]);
      }
    }
    __syncthreads();
  }
  const double ts = block_sum_d(acc_s, red);
  const double tl = block_sum_d(acc_l1, red);
  if (threadIdx.x == 0) {
    partial[2 * (size_t)blk] = ts;
    partial[2 * (size_t)blk + 1] = tl;
  }
}

__global__ __launch_bounds__(kLThreads) void k_ssim_bwd(const float *__restrict__ img,
                                                        const float *__restrict__ tgt, int B,
                                                        int H, int W, int C, Taps tp, float lam,
                                                        const float *__restrict__ pmaps,
                                                        float *__restrict__ grad) {
  __shared__ float sp[3][kLIn][kLIn];
  __shared__ float hs[3][kLIn][kLT];
  const int ntx = (W + kLT - 1) / kLT, nty = (H + kLT - 1) / kLT;
  const int blk = blockIdx.x;
  const int b = blk / (ntx * nty), t = blk % (ntx * nty);
  const int x0 = (t % ntx) * kLT, y0 = (t / ntx) * kLT;
  const size_t fo = (size_t)b * H * W * C;
  const size_t M = (size_t)B * H * W * C;
  const float invM = (float)(1.0 / (double)M);
  for (int c = 0; c < C; ++c) {
#pragma unroll
    for (int j = 0; j < 3; ++j) load_halo(sp[j], pmaps + j * M + fo, H, W, C, c, y0, x0);
    __syncthreads();
    for (int i = threadIdx.x; i < kLIn * kLT; i += kLThreads) {
      const int r = i / kLT, q = i % kLT;
      float v0 = 0.f, v1 = 0.f, v2 = 0.f;
#pragma unroll
      for (int k = 0; k < 2 * kLR + 1; ++k) {
        const float g = tp.g[k];
        v0 += g * sp[0][r][q + k];
        v1 += g * sp[1][r][q + k];
        v2 += g * sp[2][r][q + k];
      }
      hs[0][r][q] = v0;
      hs[1][r][q] = v1;
      hs[2][r][q] = v2;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kLT * kLT; i += kLThreads) {
      const int r = i / kLT, q = i % kLT;
      const int yy = y0 + r, xx = x0 + q;
      if (yy >= H || xx >= W) continue;
      float g0 = 0.f, g1 = 0.f, g2 = 0.f;
#pragma unroll
      for (int k = 0; k < 2 * kLR + 1; ++k) {
        const float g = tp.g[k];
        g0 += g * hs[0][r + k][q];
        g1 += g * hs[1][r + k][q];
        g2 += g * hs[2][r + k][q];
      }
      const size_t o = fo + ((size_t)yy * W + xx) * C + c;
      const float xv = img[o], yv = tgt[o];
      const float d = xv - yv;
      const float sg = d > 0.f ? 1.f : (d < 0.f ? -1.f : 0.f);
      grad[o] = (1.f - lam) * invM * sg - lam * invM * (g0 + 2.f * xv * g1 + yv * g2);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kLThreads) void k_loss_reduce(const double *__restrict__ partial,
                                                           int nblk, double M, double lam,
                                                           double *loss) {
  __shared__ double red[kLThreads / kWave];
  double s = 0.0, l = 0.0;
  for (int i = threadIdx.x; i < nblk; i += kLThreads) {
    s += partial[2 * (size_t)i];
    l += partial[2 * (size_t)i + 1];
  }
  const double ts = block_sum_d(s, red);
  const double tl = block_sum_d(l, red);
  if (threadIdx.x == 0) *loss = (1.0 - lam) * tl / M + lam * (1.0 - ts / M);
}

long long loss_blocks(int B, int H, int W) {
  return (long long)B * ((H + kLT - 1) / kLT) * ((W + kLT - 1) / kLT);
}

hipError_t launch_loss(const float *img, const float *tgt, int B, int H, int W, int C, float lam,
                       float c1, float c2, float *grad, double *loss, void *ws, hipStream_t st) {
  Taps tp;
  double g[2 * kLR + 1], sum = 0.0;
  for (int k = 0; k < 2 * kLR + 1; ++k) {
    const double d = k - kLR;
    g[k] = exp(-d * d / (2.0 * 1.5 * 1.5));
    sum += g[k];
  }
  for (int k = 0; k < 2 * kLR + 1; ++k) tp.g[k] = (float)(g[k] / sum);
  const long long nblk = loss_blocks(B, H, W);
  const size_t M = (size_t)B * H * W * C;
  float *pmaps = (float *)ws;
  double *partial = (double *)((char *)ws + align256(3 * M * sizeof(float)));
  PDR_TIMED(PDR_K_LOSS_FWD, st,
            hipLaunchKernelGGL(k_ssim_fwd, dim3((unsigned)nblk), dim3(kLThreads), 0, st, img, tgt,
                               B, H, W, C, tp, c1, c2, pmaps, partial));
  PDR_TIMED(PDR_K_LOSS_BWD, st,
            hipLaunchKernelGGL(k_ssim_bwd, dim3((unsigned)nblk), dim3(kLThreads), 0, st, img, tgt,
                               B, H, W, C, tp, lam, (const float *)pmaps, grad));
  PDR_TIMED(PDR_K_LOSS_REDUCE, st,
            hipLaunchKernelGGL(k_loss_reduce, dim3(1), dim3(kLThreads), 0, st,
                               (const double *)partial, (int)nblk, (double)M, (double)lam, loss));
  return hipGetLastError();
}

size_t loss_workspace_bytes(int B, int H, int W, int C) {
  const size_t M = (size_t)B * H * W * C;
  return align256(3 * M * sizeof(float)) + align256((size_t)loss_blocks(B, H, W) * 2 * sizeof(double));
}

}  // namespace pdr
