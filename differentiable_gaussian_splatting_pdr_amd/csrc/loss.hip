// loss.hip -- combined L1 + SSIM training loss of rendered frames and its
// gradient with respect to the rendered image.
//
//   loss = (1 - lam) mean|I - T| + lam (1 - mean SSIM(I, T))
//
// SSIM per frame and channel with the 11x11 Gaussian window (sigma 1.5,
// weights summing to 1), zero padding outside the frame, constants c1, c2;
// means over all M = B*H*W*C values; d|u|/du = 0 at u = 0.
//
// Both window passes use the same row walk.  A workgroup owns one frame, a
// band of pixels of one row-span and a group of cg interleaved channels
// (cg = C for C <= 16), i.e. a contiguous run of every image row: thread t
// owns flat column t of that run, whose horizontal neighbours sit at
// t +- k*cg.  The workgroup walks its rows top to bottom (plus the 5-row
// window halo on both sides), staging two rows at a time in LDS (double
// buffered, loads for the next pair in flight while the current pair is
// processed).  Each thread forms the horizontal window sums of its column
// for the new row and keeps the last 11 rows of them in registers (a ring
// indexed by the row number mod 11, resolved at compile time by a switch on
// the phase), so the vertical window sum of the row 5 above costs 11 FMAs
// per quantity and no LDS traffic.
//
// k_ssim_fwd: quantities x, y, x^2, y^2, xy (x and y staged, products
//   formed per tap, which costs less than moving them through LDS); per output value s = A1 A2 / (B1 B2) and the partial
//   derivatives of s with respect to mu_x, m_xx, m_xy, written as three
//   fp32 maps; per-workgroup fp64 sums of s and |x - y|.
// k_ssim_bwd: quantities = the three partial maps (zero outside the frame);
//   dL/dx = (1 - lam)/M sign(x - y) - lam/M [G*P_mu + 2 x G*P_xx + y G*P_xy].
// k_loss_reduce: one workgroup adds the per-workgroup sums in a fixed order.
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "pdr_common.hpp"
#include "pdr_internal.hpp"
#include "pdr_splat.h"

namespace pdr {

namespace {

constexpr int kTaps = 11;               // window taps per axis
constexpr int kHalf = 5;                // window radius
#ifndef PDR_LOSS_ROWS
#define PDR_LOSS_ROWS 2
#endif
constexpr int kLossRows = PDR_LOSS_ROWS;  // rows staged per LDS buffer (2 or 4)
static_assert(kLossRows == 2 || kLossRows == 4, "rows per chunk");
constexpr int kLossMaxThreads = 512;    // threads of a workgroup (flat columns)
constexpr int kLossMaxCg = 16;          // channels of one group
constexpr int kLossMaxL = kLossMaxThreads + 2 * kHalf * kLossMaxCg;  // staged run length
static_assert(2 * kLossRows * kLossMaxL * 12 <= 65536, "staging buffers exceed 64 KB of LDS");
#ifndef PDR_LOSS_MIN_GROUPS
#define PDR_LOSS_MIN_GROUPS 768
#endif

#ifndef PDR_LOSS_WPE
#define PDR_LOSS_WPE 1
#endif
#define PDR_LOSS_KERNEL \
  __global__ __launch_bounds__(kLossMaxThreads) __attribute__((amdgpu_waves_per_eu(PDR_LOSS_WPE)))

template <int V>
using IC = std::integral_constant<int, V>;

struct Taps {
  float g[kTaps];
};

struct LossGeom {
  int H, W, C;
  int cg;      // channels per group
  int ngrp;    // channel groups (C / cg)
  int pw;      // pixels per band
  int nb;      // bands per row
  int bw;      // threads per workgroup (multiple of 64)
  int L;       // staged run length (pw + 10) * cg
  int th;      // output rows per workgroup
  int nrb;     // row blocks per frame
  int items;   // workgroups per frame
};

int largest_divisor_upto(int C, int cap) {
  for (int d = cap < C ? cap : C; d > 1; --d)
    if (C % d == 0) return d;
  return 1;
}

LossGeom loss_geom(int B, int H, int W, int C) {
  LossGeom g;
  g.H = H;
  g.W = W;
  g.C = C;
  g.cg = C <= kLossMaxCg ? C : largest_divisor_upto(C, kLossMaxCg);
  g.ngrp = C / g.cg;
  const int pwmax = kLossMaxThreads / g.cg;
  g.nb = (W + pwmax - 1) / pwmax;
  g.pw = (W + g.nb - 1) / g.nb;
  g.L = (g.pw + 2 * kHalf) * g.cg;
  int bw = (g.pw * g.cg + kWave - 1) / kWave * kWave;
  const int half = ((g.L + 1) / 2 + kWave - 1) / kWave * kWave;  // at most two staged slots
  g.bw = bw > half ? bw : half;
  g.th = 64;
  while (g.th > 16 &&
         (long long)B * g.ngrp * g.nb * ((H + g.th - 1) / g.th) < PDR_LOSS_MIN_GROUPS)
    g.th /= 2;
  g.nrb = (H + g.th - 1) / g.th;
  g.items = g.ngrp * g.nb * g.nrb;
  return g;
}

struct BlockPos {
  int b, x0, npx, c0, y0, yend;
};

// Workgroup -> (frame, band, channel group, row block); frames are spread
// over the 8 XCDs so that the row blocks of one frame (which share halo
// rows) run under the same L2.
__device__ __forceinline__ bool block_pos(const LossGeom &g, int B, BlockPos *p, int *lin) {
  int b, item;
  if (!xcd_frame_item(blockIdx.x, g.items, B, &b, &item)) return false;
  *lin = b * g.items + item;
  const int rb = item % g.nrb;
  const int rest = item / g.nrb;
  const int band = rest % g.nb;
  const int grp = rest / g.nb;
  p->b = b;
  p->x0 = band * g.pw;
  p->npx = min(g.pw, g.W - p->x0);
  p->c0 = grp * g.cg;
  p->y0 = rb * g.th;
  p->yend = min(p->y0 + g.th, g.H);
  return true;
}

__device__ __forceinline__ double block_sum_d(double v, double *red) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  double t = 0.0;
  const int nw = blockDim.x >> 6;
  for (int w = 0; w < nw; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Frame-sized buffer resources: loads past num_records return 0 and
// stores past it are dropped, which gives the zero padding and the
// column masking without branches.  Byte offsets are 32-bit (frames hold
// fewer than 2^29 values, so an offset of kOut plus a row offset never
// wraps).
constexpr uint32_t kOut = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t frame_res(const float *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// (the b32 builtins move raw 32-bit words: reinterpret, never convert)
__device__ __forceinline__ float ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, float v, uint32_t voff,
                                   uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)voff, (int)soff,
                                        0);
}

// Byte offsets (within one image row) of the two staged slots of this
// thread, kOut outside the frame or past the run.
__device__ __forceinline__ void slot_offsets(const LossGeom &g, const BlockPos &p, uint32_t off[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = threadIdx.x + j * g.bw;
    off[j] = kOut;
    if (e < g.L) {
      const int px = p.x0 - kHalf + e / g.cg;
      const int ch = p.c0 + e % g.cg;
      if (px >= 0 && px < g.W) off[j] = (uint32_t)(px * g.C + ch) * 4u;
    }
  }
}

template <int CG>
__device__ __forceinline__ int tap_stride(int cg) {
  return CG > 0 ? CG : cg;
}

// Per-thread walk set-up shared by both passes.
struct Walk {
  int T;          // rows walked: output rows + 10
  int nch;        // staged chunks
  int ybase;      // image row of walk step 0
  uint32_t rowb;  // bytes per image row
  uint32_t ocol;  // byte offset of this thread's output column, kOut if none
  bool has_col;
};

__device__ __forceinline__ Walk make_walk(const LossGeom &g, const BlockPos &p) {
  Walk w;
  const int tid = threadIdx.x;
  w.T = (p.yend - p.y0) + 2 * kHalf;
  w.nch = (w.T + kLossRows - 1) / kLossRows;
  w.ybase = p.y0 - kHalf;
  w.rowb = (uint32_t)g.W * g.C * 4u;
  w.has_col = tid < p.npx * g.cg;
  w.ocol = w.has_col ? (uint32_t)((p.x0 + tid / g.cg) * g.C + p.c0 + tid % g.cg) * 4u : kOut;
  return w;
}

// ---------------------------------------------------------------- forward

struct FwdOut {
  __amdgpu_buffer_rsrc_t r0, r1, r2;
  bool keep;      // the thread has an output column (else its sums read
                  // LDS past the staged run and are discarded)
  double acc_s;
};

// One row of the walk at ring phase J: horizontal sums of the new row into
// ring slot J; if emit, the vertical sums of the row 5 above and its SSIM
// and partial derivatives (stored at byte offsets voff + soff).
template <int CG, int J>
__device__ __forceinline__ void fwd_step(float (&h)[kTaps][5], const float2 *__restrict__ rq,
                                         int cg, const Taps &tp, bool emit, float c1, float c2,
                                         uint32_t voff, uint32_t soff, FwdOut &out) {
  const int cs = tap_stride<CG>(cg);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f, a4 = 0.f;
#pragma unroll
  for (int k = 0; k < kTaps; ++k) {
    // products formed here: two more VALU ops per tap, 2.5x less LDS traffic
    const float2 q = rq[k * cs];
    const float wx = tp.g[k] * q.x, wy = tp.g[k] * q.y;
    a0 += wx;
    a1 += wy;
    a2 = fmaf(wx, q.x, a2);
    a3 = fmaf(wy, q.y, a3);
    a4 = fmaf(wx, q.y, a4);
  }
  h[J][0] = a0;
  h[J][1] = a1;
  h[J][2] = a2;
  h[J][3] = a3;
  h[J][4] = a4;
  if (!emit) return;
  float m[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kTaps; ++k) {
    const float w = tp.g[k];
#pragma unroll
    for (int q = 0; q < 5; ++q) m[q] = fmaf(w, h[(J + 1 + k) % kTaps][q], m[q]);
  }
  const float mx = m[0], my = m[1];
  const float mxy = mx * my;
  const float A1 = 2.f * mxy + c1;
  const float A2 = 2.f * (m[4] - mxy) + c2;
  const float B1 = mx * mx + my * my + c1;
  const float B2 = (m[2] - mx * mx) + (m[3] - my * my) + c2;
  const float ib1 = __builtin_amdgcn_rcpf(B1);
  const float ib2 = __builtin_amdgcn_rcpf(B2);
  const float ib12 = ib1 * ib2;
  const float s = A1 * A2 * ib12;
  st(out.r0, 2.f * my * (A2 - A1) * ib12 - 2.f * mx * s * (ib1 - ib2), voff, soff);
  st(out.r1, -s * ib2, voff, soff);
  st(out.r2, 2.f * A1 * ib12, voff, soff);
  out.acc_s += out.keep ? (double)s : 0.0;
}

template <int CG>
PDR_LOSS_KERNEL void k_ssim_fwd(
    const float *__restrict__ img, const float *__restrict__ tgt, int B, LossGeom g, Taps tp,
    float c1, float c2, float *__restrict__ pmaps, size_t M, double *__restrict__ partial) {
  extern __shared__ float2 lds_f2[];
  BlockPos p;
  int lin;
  if (!block_pos(g, B, &p, &lin)) return;
  __shared__ double red[kLossMaxThreads / kWave];
  const int tid = threadIdx.x;
  const int L = g.L;
  float2 *q2 = lds_f2;   // per buffer: kLossRows rows of float2 {x, y}
  const size_t fo = (size_t)p.b * g.H * g.W * g.C;
  const uint32_t fbytes = (uint32_t)g.H * g.W * g.C * 4u;
  const __amdgpu_buffer_rsrc_t rx = frame_res(img + fo, fbytes), ry = frame_res(tgt + fo, fbytes);
  uint32_t off[2];
  slot_offsets(g, p, off);
  const Walk w = make_walk(g, p);
  FwdOut out{frame_res(pmaps + fo, fbytes), frame_res(pmaps + M + fo, fbytes),
             frame_res(pmaps + 2 * M + fo, fbytes), w.has_col, 0.0};
  double acc_l1 = 0.0;

  // the next chunk: loads in flight while this chunk's rows are processed
  float pre_x[kLossRows][2], pre_y[kLossRows][2];
  auto load_chunk = [&](float (&dx)[kLossRows][2], float (&dy)[kLossRows][2], int ch) {
#pragma unroll
    for (int r = 0; r < kLossRows; ++r) {
      const int y = w.ybase + ch * kLossRows + r;
      const bool rv = y >= 0 && y < g.H;   // uniform
      const uint32_t so = rv ? (uint32_t)y * w.rowb : 0u;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t vo = rv ? off[j] : kOut;
        dx[r][j] = ld(rx, vo, so);
        dy[r][j] = ld(ry, vo, so);
      }
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int r = 0; r < kLossRows; ++r) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = tid + j * g.bw;
        if (e < L) q2[(buf * kLossRows + r) * L + e] = make_float2(pre_x[r][j], pre_y[r][j]);
      }
    }
  };

  float h[kTaps][5];
#pragma unroll
  for (int k = 0; k < kTaps; ++k)
#pragma unroll
    for (int q = 0; q < 5; ++q) h[k][q] = 0.f;

  // one row of the walk: t = row index, J = t mod 11 (compile time)
  auto row = [&](auto Jc, int t, int buf, int r) {
    if (t >= w.T) return;
    const float2 *rq = q2 + (buf * kLossRows + r) * L + tid;
    const int yin = w.ybase + t;   // row entering the ring
    if (yin >= p.y0 && yin < p.yend) {
      const float2 c = rq[kHalf * tap_stride<CG>(g.cg)];
      acc_l1 += out.keep ? (double)fabsf(c.x - c.y) : 0.0;
    }
    const bool emit = t >= 2 * kHalf;   // row yin - 5 completes
    const uint32_t so = emit ? (uint32_t)(yin - kHalf) * w.rowb : 0u;
    fwd_step<CG, decltype(Jc)::value>(h, rq, g.cg, tp, emit, c1, c2, w.ocol, so, out);
  };
  // one staged chunk of kLossRows rows; the 11 chunks of an outer
  // iteration cover 11 kLossRows rows, so every ring phase is a compile-time
  // constant
  auto chunk = [&](auto Cc, int ch0) {
    constexpr int c = decltype(Cc)::value;
    const int ch = ch0 + c;
    if (ch >= w.nch) return;
    const int buf = ch & 1;
    if (ch + 1 < w.nch) load_chunk(pre_x, pre_y, ch + 1);
    row(IC<(kLossRows * c) % kTaps>{}, kLossRows * ch, buf, 0);
    row(IC<(kLossRows * c + 1) % kTaps>{}, kLossRows * ch + 1, buf, 1);
    if constexpr (kLossRows == 4) {
      row(IC<(kLossRows * c + 2) % kTaps>{}, kLossRows * ch + 2, buf, 2);
      row(IC<(kLossRows * c + 3) % kTaps>{}, kLossRows * ch + 3, buf, 3);
    }
    if (ch + 1 < w.nch) store_chunk(buf ^ 1);
    __syncthreads();
  };

  load_chunk(pre_x, pre_y, 0);
  store_chunk(0);
  __syncthreads();
  for (int ch0 = 0; ch0 < w.nch; ch0 += kTaps) {
    chunk(IC<0>{}, ch0);
    chunk(IC<1>{}, ch0);
    chunk(IC<2>{}, ch0);
    chunk(IC<3>{}, ch0);
    chunk(IC<4>{}, ch0);
    chunk(IC<5>{}, ch0);
    chunk(IC<6>{}, ch0);
    chunk(IC<7>{}, ch0);
    chunk(IC<8>{}, ch0);
    chunk(IC<9>{}, ch0);
    chunk(IC<10>{}, ch0);
  }
  const double ts = block_sum_d(out.acc_s, red);
  const double tl = block_sum_d(acc_l1, red);
  if (tid == 0) {
    partial[2 * (size_t)lin] = ts;
    partial[2 * (size_t)lin + 1] = tl;
  }
}

// --------------------------------------------------------------- backward

template <int CG, int J>
__device__ __forceinline__ void bwd_step(float (&h)[kTaps][3], const float2 *__restrict__ rq,
                                         const float *__restrict__ rs, int cg, const Taps &tp,
                                         bool emit, float xo, float yo, float wl1, float wss,
                                         __amdgpu_buffer_rsrc_t rg, uint32_t voff, uint32_t soff) {
  const int cs = tap_stride<CG>(cg);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f;
#pragma unroll
  for (int k = 0; k < kTaps; ++k) {
    const float2 q = rq[k * cs];
    const float q2 = rs[k * cs];
    const float w = tp.g[k];
    a0 = fmaf(w, q.x, a0);
    a1 = fmaf(w, q.y, a1);
    a2 = fmaf(w, q2, a2);
  }
  h[J][0] = a0;
  h[J][1] = a1;
  h[J][2] = a2;
  if (!emit) return;
  float m0 = 0.f, m1 = 0.f, m2 = 0.f;
#pragma unroll
  for (int k = 0; k < kTaps; ++k) {
    const float w = tp.g[k];
    m0 = fmaf(w, h[(J + 1 + k) % kTaps][0], m0);
    m1 = fmaf(w, h[(J + 1 + k) % kTaps][1], m1);
    m2 = fmaf(w, h[(J + 1 + k) % kTaps][2], m2);
  }
  const float d = xo - yo;
  const float sg = d > 0.f ? 1.f : (d < 0.f ? -1.f : 0.f);
  st(rg, wl1 * sg - wss * (m0 + 2.f * xo * m1 + yo * m2), voff, soff);
}

template <int CG>
PDR_LOSS_KERNEL void k_ssim_bwd(
    const float *__restrict__ img, const float *__restrict__ tgt, int B, LossGeom g, Taps tp,
    float wl1, float wss, const float *__restrict__ pmaps, size_t M, float *__restrict__ grad) {
  extern __shared__ float2 lds_f2[];
  BlockPos p;
  int lin;
  if (!block_pos(g, B, &p, &lin)) return;
  const int tid = threadIdx.x;
  const int L = g.L;
  // per buffer: kLossRows rows of float2 {P_mu, P_xx}; then all rows of P_xy
  float2 *q2 = lds_f2;
  float *qs = (float *)(lds_f2 + 2 * kLossRows * L);
  const size_t fo = (size_t)p.b * g.H * g.W * g.C;
  const uint32_t fbytes = (uint32_t)g.H * g.W * g.C * 4u;
  const __amdgpu_buffer_rsrc_t r0 = frame_res(pmaps + fo, fbytes),
                               r1 = frame_res(pmaps + M + fo, fbytes),
                               r2 = frame_res(pmaps + 2 * M + fo, fbytes);
  const __amdgpu_buffer_rsrc_t rx = frame_res(img + fo, fbytes), ry = frame_res(tgt + fo, fbytes),
                               rg = frame_res(grad + fo, fbytes);
  uint32_t off[2];
  slot_offsets(g, p, off);
  const Walk w = make_walk(g, p);

  float pre[kLossRows][2][3];
  auto load_chunk = [&](float (&d)[kLossRows][2][3], int ch) {
#pragma unroll
    for (int r = 0; r < kLossRows; ++r) {
      const int y = w.ybase + ch * kLossRows + r;
      const bool rv = y >= 0 && y < g.H;   // uniform
      const uint32_t so = rv ? (uint32_t)y * w.rowb : 0u;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t vo = rv ? off[j] : kOut;
        d[r][j][0] = ld(r0, vo, so);
        d[r][j][1] = ld(r1, vo, so);
        d[r][j][2] = ld(r2, vo, so);
      }
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int r = 0; r < kLossRows; ++r) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = tid + j * g.bw;
        if (e < L) {
          const int i = (buf * kLossRows + r) * L + e;
          q2[i] = make_float2(pre[r][j][0], pre[r][j][1]);
          qs[i] = pre[r][j][2];
        }
      }
    }
  };

  float h[kTaps][3];
#pragma unroll
  for (int k = 0; k < kTaps; ++k)
#pragma unroll
    for (int q = 0; q < 3; ++q) h[k][q] = 0.f;

  auto row = [&](auto Jc, int t, int buf, int r, float xo, float yo) {
    if (t >= w.T) return;
    const int ri = (buf * kLossRows + r) * L + tid;
    const bool emit = t >= 2 * kHalf;
    const uint32_t so = emit ? (uint32_t)(w.ybase + t - kHalf) * w.rowb : 0u;
    bwd_step<CG, decltype(Jc)::value>(h, q2 + ri, qs + ri, g.cg, tp, emit, xo, yo, wl1, wss, rg,
                                      w.ocol, so);
  };
  auto chunk = [&](auto Cc, int ch0) {
    constexpr int c = decltype(Cc)::value;
    const int ch = ch0 + c;
    if (ch >= w.nch) return;
    const int buf = ch & 1;
    // image and target at this chunk's output rows
    float xo[kLossRows], yo[kLossRows];
#pragma unroll
    for (int r = 0; r < kLossRows; ++r) {
      const int t = ch * kLossRows + r;
      const bool v = t >= 2 * kHalf && t < w.T;   // uniform
      const uint32_t so = v ? (uint32_t)(w.ybase + t - kHalf) * w.rowb : 0u;
      const uint32_t vo = v ? w.ocol : kOut;
      xo[r] = ld(rx, vo, so);
      yo[r] = ld(ry, vo, so);
    }
    if (ch + 1 < w.nch) load_chunk(pre, ch + 1);
    row(IC<(kLossRows * c) % kTaps>{}, kLossRows * ch, buf, 0, xo[0], yo[0]);
    row(IC<(kLossRows * c + 1) % kTaps>{}, kLossRows * ch + 1, buf, 1, xo[1], yo[1]);
    if constexpr (kLossRows == 4) {
      row(IC<(kLossRows * c + 2) % kTaps>{}, kLossRows * ch + 2, buf, 2, xo[2], yo[2]);
      row(IC<(kLossRows * c + 3) % kTaps>{}, kLossRows * ch + 3, buf, 3, xo[3], yo[3]);
    }
    if (ch + 1 < w.nch) store_chunk(buf ^ 1);
    __syncthreads();
  };

  load_chunk(pre, 0);
  store_chunk(0);
  __syncthreads();
  for (int ch0 = 0; ch0 < w.nch; ch0 += kTaps) {
    chunk(IC<0>{}, ch0);
    chunk(IC<1>{}, ch0);
    chunk(IC<2>{}, ch0);
    chunk(IC<3>{}, ch0);
    chunk(IC<4>{}, ch0);
    chunk(IC<5>{}, ch0);
    chunk(IC<6>{}, ch0);
    chunk(IC<7>{}, ch0);
    chunk(IC<8>{}, ch0);
    chunk(IC<9>{}, ch0);
    chunk(IC<10>{}, ch0);
  }
}

__global__ __launch_bounds__(256) void k_loss_reduce(const double *__restrict__ partial, int nblk,
                                                     double M, double lam, double *loss) {
  __shared__ double red[256 / kWave];
  double s = 0.0, l = 0.0;
  for (int i = threadIdx.x; i < nblk; i += 256) {
    s += partial[2 * (size_t)i];
    l += partial[2 * (size_t)i + 1];
  }
  const double ts = block_sum_d(s, red);
  const double tl = block_sum_d(l, red);
  if (threadIdx.x == 0) *loss = (1.0 - lam) * tl / M + lam * (1.0 - ts / M);
}

template <int CG>
void launch_cg(const float *img, const float *tgt, int B, const LossGeom &g, const Taps &tp,
               float c1, float c2, float wl1, float wss, float *pmaps, size_t M, double *partial,
               float *grad, hipStream_t st) {
  const dim3 grid((unsigned)xcd_grid(g.items, B)), block((unsigned)g.bw);
  const size_t lds_f = (size_t)2 * kLossRows * g.L * sizeof(float2);
  const size_t lds_b = (size_t)2 * kLossRows * g.L * (sizeof(float2) + sizeof(float));
  PDR_TIMED(PDR_K_LOSS_FWD, st,
            hipLaunchKernelGGL(k_ssim_fwd<CG>, grid, block, lds_f, st, img, tgt, B, g, tp, c1, c2,
                               pmaps, M, partial));
  PDR_TIMED(PDR_K_LOSS_BWD, st,
            hipLaunchKernelGGL(k_ssim_bwd<CG>, grid, block, lds_b, st, img, tgt, B, g, tp, wl1, wss,
                               (const float *)pmaps, M, grad));
}

}  // namespace

hipError_t launch_loss(const float *img, const float *tgt, int B, int H, int W, int C, float lam,
                       float c1, float c2, float *grad, double *loss, void *ws, hipStream_t st) {
  Taps tp;
  double gw[kTaps], sum = 0.0;
  for (int k = 0; k < kTaps; ++k) {
    const double d = k - kHalf;
    gw[k] = exp(-d * d / (2.0 * 1.5 * 1.5));
    sum += gw[k];
  }
  for (int k = 0; k < kTaps; ++k) tp.g[k] = (float)(gw[k] / sum);
  const LossGeom g = loss_geom(B, H, W, C);
  const size_t M = (size_t)B * H * W * C;
  float *pmaps = (float *)ws;
  double *partial = (double *)((char *)ws + align256(3 * M * sizeof(float)));
  const float wl1 = (float)((1.0 - (double)lam) / (double)M);
  const float wss = (float)((double)lam / (double)M);
  switch (g.cg) {
    case 1: launch_cg<1>(img, tgt, B, g, tp, c1, c2, wl1, wss, pmaps, M, partial, grad, st); break;
    case 2: launch_cg<2>(img, tgt, B, g, tp, c1, c2, wl1, wss, pmaps, M, partial, grad, st); break;
    case 3: launch_cg<3>(img, tgt, B, g, tp, c1, c2, wl1, wss, pmaps, M, partial, grad, st); break;
    case 4: launch_cg<4>(img, tgt, B, g, tp, c1, c2, wl1, wss, pmaps, M, partial, grad, st); break;
    case 8: launch_cg<8>(img, tgt, B, g, tp, c1, c2, wl1, wss, pmaps, M, partial, grad, st); break;
    case 16: launch_cg<16>(img, tgt, B, g, tp, c1, c2, wl1, wss, pmaps, M, partial, grad, st); break;
    default: launch_cg<0>(img, tgt, B, g, tp, c1, c2, wl1, wss, pmaps, M, partial, grad, st); break;
  }
  const int nblk = B * g.items;
  PDR_TIMED(PDR_K_LOSS_REDUCE, st,
            hipLaunchKernelGGL(k_loss_reduce, dim3(1), dim3(256), 0, st, (const double *)partial,
                               nblk, (double)M, (double)lam, loss));
  return hipGetLastError();
}

size_t loss_workspace_bytes(int B, int H, int W, int C) {
  const size_t M = (size_t)B * H * W * C;
  const LossGeom g = loss_geom(B, H, W, C);
  return align256(3 * M * sizeof(float)) + align256((size_t)B * g.items * 2 * sizeof(double));
}

}  // namespace pdr
