// span.hip -- tile-free backward: one wave per Gaussian over the compacted
// pixels of its support.
//
// The tile backward evaluates every pixel of every 8x8 unit that a
// Gaussian's truncated ellipse may touch (under half of those lanes are
// inside the support on the benchmark workload) and reduces the per-lane
// partial sums once per (tile, Gaussian) list entry.  Here a wave owns one Gaussian: for every row of its box it
// computes the row's span of pixel centres inside the truncated ellipse
// (the roots of a quadratic, widened by a relative 1e-3 of the threshold so
// the span is a superset; the per-pixel test q <= k^2 then decides exactly as
// in the tile kernels), packs the spans of up to 64 rows back to back, and
// walks them 64 pixels at a time, so nearly every lane evaluates a pixel of
// the support.  dL/dI is read straight from memory (coalesced along the
// spans, L2-resident per frame).  The per-lane partial sums are reduced once
// per Gaussian, and the wave applies the chain rule and stores the gradient
// row itself: no atomics, no zeroing pass, no separate finalisation.
//
// Pixel -> (row, column) within a window of 64 packed pixels: every row
// whose span starts inside the window writes its index at that start in a
// per-wave LDS array; an inclusive max-scan over the lanes then gives every
// lane its row, with the last row of the previous window carried in.
//
// The page 3 prior art ("contour-based differentiable rendering", first
// paragraph) pairs tile-free splat processing with subgroup gradient
// reduction; this is that idea on wave64 for the 2D, order-free sums here.
#include <math.h>
#include <stdint.h>

#include "pdr_common.hpp"
#include "pdr_internal.hpp"
#include "pdr_splat.h"

namespace pdr {

namespace {

constexpr int kSpanThreads = 256;                   // four waves
constexpr int kSpanWaves = kSpanThreads / kWave;
constexpr int kSpanPerWave = 4;                     // Gaussians per wave, in turn
constexpr int kSpanPerBlock = kSpanWaves * kSpanPerWave;
constexpr float kSpanMargin = 1.0e-3f;              // relative widening of the span threshold

__device__ __forceinline__ int wave_incl_max(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, kDppRowShr1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, kDppRowShr2, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, kDppRowShr4, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, kDppRowShr8, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, kDppRowBcast15, 0xA, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(-1, v, kDppRowBcast31, 0xC, 0xF, false));
  return v;
}

// dL/dI of one frame through a buffer resource: 32-bit byte offsets, and an
// offset past the frame (kOff) reads 0 (a lane with no pixel).  GB is the
// format's bytes per value.
constexpr uint32_t kOff = 0x80000000u;

template <int FMT>
__device__ __forceinline__ float load_gb(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (FMT == PDR_FMT_F32) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
  } else {
    const unsigned short b = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    if constexpr (FMT == PDR_FMT_F16) return (float)__builtin_bit_cast(_Float16, b);
    else return (float)__builtin_bit_cast(__bf16, b);
  }
}


template <int K>
struct SpanPow2 {
  static constexpr int value = K <= 8 ? 8 : (K <= 16 ? 16 : 32);
};

template <int CP, int FMT>
__global__ __launch_bounds__(kSpanThreads) void k_backward_span(
    const GRec *__restrict__ recs, const ThinRec *__restrict__ thin,
    const float *__restrict__ params, const void *__restrict__ gimg,
    int B, int N, int H, int W, int C, float thr, int items, float *__restrict__ grad,
    const WsHeader *hdr) {
  constexpr int K = CP + 5;
  constexpr int KP = SpanPow2<K>::value;
  constexpr int GB = FMT == PDR_FMT_F32 ? 4 : 2;
  __shared__ int s_start[kSpanWaves][kWave];
  __shared__ int s_xs[kSpanWaves][kWave];
  __shared__ int s_row[kSpanWaves][kWave];
  __shared__ float s_sum[kSpanWaves][KP];
  int f, item;
  if (!xcd_frame_item(blockIdx.x, items, B, &f, &item)) return;
  // binning that overflowed, or records that are not this call's: every
  // gradient of the call is set to NaN
  const bool bad = (hdr->status & (kStatusOverflow | kStatusStale)) != 0;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int P = 5 + C;
  const float thr_span = thr * (1.0f + kSpanMargin);
  int *st_start = s_start[wv], *st_xs = s_xs[wv], *st_row = s_row[wv];
  float *st_sum = s_sum[wv];
  const int vidx = value_index<KP>(lane);

  for (int j = 0; j < kSpanPerWave; ++j) {
    const int n = item * kSpanPerBlock + j * kSpanWaves + wv;
    if (n >= N) break;
    const size_t gi = (size_t)f * N + n;
    float *out = grad + gi * P;
    if (bad) {
      for (int c = lane; c < P; c += kWave) out[c] = __builtin_nanf("");
      continue;
    }
    const GRec r = recs[gi];
    const int x0 = (int)(r.bx & 0xFFFFu), x1 = (int)(r.bx >> 16);
    const int y0 = (int)(r.by & 0xFFFFu), y1 = (int)(r.by >> 16);
    if (x0 > x1 || y0 > y1) {   // culled or off-screen: zero gradient
      for (int c = lane; c < P; c += kWave) out[c] = 0.f;
      continue;
    }
    const float *pg = params + gi * P;
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(gimg)) + (size_t)f * H * W * C * GB, (short)0,
        (int)((uint32_t)H * (uint32_t)W * (uint32_t)(C * GB)), 0x00020000);
    float a[CP];
#pragma unroll
    for (int c = 0; c < CP; ++c) a[c] = c < C ? pg[5 + c] : 0.f;
    float part[KP];
#pragma unroll
    for (int k = 0; k < KP; ++k) part[k] = 0.f;
    // The row's span in closed form: with d = p - mu,
    //   q(dx) = qa (dx - xc)^2 + qd dy^2,  xc = -(qb / qa) dy,  qd = det^2 / qa
    // (qa = l11^2 + l21^2, qb = l11 l12 + l21 l22, det = l11 l22 - l12 l21, a
    // sum of two terms of one sign), which loses nothing to cancellation
    // where the expanded quadratic's discriminant loses u |L|^2 |d|^2 for
    // thin Gaussians.  The span is widened by the rounding of its centre.
    const float qa = r.l11 * r.l11 + r.l21 * r.l21;
    const float qb = r.l11 * r.l12 + r.l21 * r.l22;
    const float qc = r.l12 * r.l12 + r.l22 * r.l22;
    const float det = r.l11 * r.l22 - r.l12 * r.l21;
    const float inv_qa = 1.0f / qa;
    const float xb = qb * inv_qa, qd = det * det * inv_qa;
    const float xb_err = 2.4e-7f * sqrtf(qc * inv_qa);   // 4u sqrt(qc / qa) bounds |xb| rounding / |dy|
    // a thin Gaussian takes the compensated evaluation about its split mean
    // (rows in thin-row-last order; the sums of swapped rows trade places)
    const bool thin_g = is_thin(r.l11, r.l12, r.l21, r.l22) && (thin[gi].flags & kThinOk);
    ThinX tx{};
    float l11 = r.l11, l12 = r.l12, l21 = r.l21, l22 = r.l22, mx = r.mx, my = r.my;
    bool sw = false;
    if (thin_g) {
      const ThinRec tr = thin[gi];
      sw = (tr.flags & kThinSwap) != 0;
      if (sw) {
        l11 = r.l21; l12 = r.l22; l21 = r.l11; l22 = r.l12;
      }
      mx = tr.mhx;
      my = tr.mhy;
      tx = ThinX{tr.lo21, tr.lo22, tr.c1, tr.c2};
    }

    for (int ry = y0; ry <= y1; ry += kWave) {
      const int y = ry + lane;
      int len = 0, xs = 0;
      if (y <= y1) {
        const float dy = ((float)y + 0.5f) - r.my;
        const float rem = thr_span - qd * dy * dy;
        if (rem >= 0.f) {
          const float half = sqrtf(rem * inv_qa);
          const float xc = r.mx - xb * dy - 0.5f;
          const float pad = 1e-3f + xb_err * fabsf(dy) + 2.4e-7f * (fabsf(xc) + half);
          const float lo = xc - half - pad, hi = xc + half + pad;
          xs = max(x0, (int)ceilf(lo));
          const int xe = min(x1, (int)floorf(hi));
          len = max(0, xe - xs + 1);
        }
      }
      const int incl = wave_incl_scan(len);
      const int excl = incl - len;
      const int total = __builtin_amdgcn_readlane(incl, 63);
      __asm__ volatile("" ::: "memory");
      st_start[lane] = excl;
      st_xs[lane] = xs;
      int carry = 0;
      // this lane's pixel of the window starting at packed index base:
      // (x, row offset) and the byte offset of its dL/dI (kOff when none)
      auto map_window = [&](int base, int *px, int *prow) -> uint32_t {
        // lanes exchange values through the per-wave LDS arrays below: keep
        // the compiler from forwarding a lane's own stores to its loads
        __asm__ volatile("" ::: "memory");
        st_row[lane] = -1;
        __asm__ volatile("" ::: "memory");
        if (len > 0 && excl >= base && excl < base + kWave) st_row[excl - base] = lane;
        __asm__ volatile("" ::: "memory");
        int rl = wave_incl_max(st_row[lane]);
        rl = rl < 0 ? carry : rl;
        carry = __builtin_amdgcn_readlane(rl, 63);
        const int p = base + lane;
        const int x = st_xs[rl] + (p - st_start[rl]);
        *px = x;
        *prow = rl;
        return p < total ? ((uint32_t)(ry + rl) * (uint32_t)W + (uint32_t)x) * (uint32_t)(C * GB)
                         : kOff;
      };
      auto load_window = [&](uint32_t off, float (&G)[CP]) {
#pragma unroll
        for (int c = 0; c < CP; ++c) {
          // CP == C up to 4 channels; above, CP is padded and the padding reads nothing
          if constexpr (CP > 4) {
            if (c >= C) {
              G[c] = 0.f;
              continue;
            }
          }
          G[c] = load_gb<FMT>(rg, off + (uint32_t)(c * GB));
        }
      };
      int x_c, row_c;
      uint32_t off_c = map_window(0, &x_c, &row_c);
      float G_c[CP];
      load_window(off_c, G_c);
      for (int base = 0; base < total; base += kWave) {
        // the next window's mapping and loads go out before this window's math
        int x_n = 0, row_n = 0;
        uint32_t off_n = kOff;
        float G_n[CP];
        if (base + kWave < total) {
          off_n = map_window(base + kWave, &x_n, &row_n);
          load_window(off_n, G_n);
        }
        if (off_c != kOff) {
          const float dx = ((float)x_c + 0.5f) - mx;   // exact about a split mean
          const float dy = ((float)(ry + row_c) + 0.5f) - my;
          float u1, u2;
          if (thin_g) whiten<true>(l11, l12, l21, l22, tx, dx, dy, u1, u2);
          else whiten<false>(l11, l12, l21, l22, tx, dx, dy, u1, u2);
          const float q = u1 * u1 + u2 * u2;
          if (q <= thr) {
            const float w = __builtin_amdgcn_exp2f(-q);
            float h = 0.f;
#pragma unroll
            for (int c = 0; c < CP; ++c) h += G_c[c] * a[c];
            const float v = h * w;
#pragma unroll
            for (int c = 0; c < CP; ++c) part[c] += G_c[c] * w;
            const float t1 = v * u1, t2 = v * u2;
            part[CP + 0] += t1;
            part[CP + 1] += t2;
            part[CP + 2] += t1 * u1;
            part[CP + 3] += t2 * u2;
            part[CP + 4] += t1 * u2;
          }
        }
        x_c = x_n;
        row_c = row_n;
        off_c = off_n;
#pragma unroll
        for (int c = 0; c < CP; ++c) G_c[c] = G_n[c];
      }
    }
    const float tot = wave_reduce_transposed<KP>(part, lane);
    // swapped rows accumulated (S2, S1, S22, S11, S12): back to row order
    const int vs = (sw && vidx >= CP && vidx < CP + 4) ? CP + ((vidx - CP) ^ 1) : vidx;
    if (reduce_issuer<KP>(lane)) st_sum[vs] = tot;
    // the chain rule (fp64), undoing the kappa scale of the whitened rows:
    //   dmu = L^T (S1, S2), ds1 = S11 / s1, ds2 = S22 / s2,
    //   dtheta = (s1/s2 - s2/s1) S12, da = A
    __asm__ volatile("" ::: "memory");   // other lanes' sums are read below
    if (lane < P) {
      const double k2 = kKappa2;   // kappa^2
      float o;
      if (lane >= 5) {
        o = st_sum[lane - 5];
      } else {
        const double S1 = st_sum[CP], S2 = st_sum[CP + 1], S11 = st_sum[CP + 2],
                     S22 = st_sum[CP + 3], S12 = st_sum[CP + 4];
        const double s1 = pg[2], s2 = pg[3];
        double v;
        if (lane == 0) v = ((double)r.l11 * S1 + (double)r.l21 * S2) / k2;
        else if (lane == 1) v = ((double)r.l12 * S1 + (double)r.l22 * S2) / k2;
        else if (lane == 2) v = S11 / (k2 * s1);
        else if (lane == 3) v = S22 / (k2 * s2);
        else v = ((s1 * s1 - s2 * s2) / (s1 * s2)) * S12 / k2;
        o = (float)v;
      }
      out[lane] = o;
    }
  }
}

// Clear the stale bit and, when the backward reuses the forward's
// preprocessing, check the workspace stamp against this call's arguments.
__global__ void k_span_stamp(WsHeader *hdr, int check, int B, int N, int H, int W, int C,
                             float radius, unsigned long long ptr) {
  if (threadIdx.x != 0) return;
  // without reuse the records were just rebuilt and no lists are involved
  int st = check ? (hdr->status & ~kStatusStale) : 0;
  if (check) {
    const bool same = hdr->stamp[0] == B && hdr->stamp[1] == N && hdr->stamp[2] == H &&
                      hdr->stamp[3] == W && hdr->stamp[4] == C &&
                      hdr->stamp[5] == __float_as_int(radius) &&
                      hdr->stamp[6] == (int)(unsigned)(ptr & 0xffffffffull) &&
                      hdr->stamp[7] == (int)(unsigned)(ptr >> 32);
    if (!same) st |= kStatusStale;
  }
  hdr->status = st;
}

template <int CP, int FMT>
void launch_span_fmt(const GRec *recs, const ThinRec *thin, const float *params, const void *gimg,
                     int B, int N, int H, int W, int C, float thr, float *grad, const WsHeader *hdr,
                     hipStream_t st) {
  const int items = (N + kSpanPerBlock - 1) / kSpanPerBlock;
  PDR_TIMED(PDR_K_BACKWARD_RASTER, st,
            hipLaunchKernelGGL((k_backward_span<CP, FMT>), dim3((unsigned)xcd_grid(items, B)),
                               dim3(kSpanThreads), 0, st, recs, thin, params, gimg, B, N, H, W, C,
                               thr, items, grad, hdr));
}

template <int CP>
void launch_span_cp(const GRec *recs, const ThinRec *thin, const float *params, const void *gimg,
                    int fmt, int B, int N, int H, int W, int C, float thr, float *grad,
                    const WsHeader *hdr, hipStream_t st) {
  if (fmt == PDR_FMT_F16)
    launch_span_fmt<CP, PDR_FMT_F16>(recs, thin, params, gimg, B, N, H, W, C, thr, grad, hdr, st);
  else if (fmt == PDR_FMT_BF16)
    launch_span_fmt<CP, PDR_FMT_BF16>(recs, thin, params, gimg, B, N, H, W, C, thr, grad, hdr, st);
  else
    launch_span_fmt<CP, PDR_FMT_F32>(recs, thin, params, gimg, B, N, H, W, C, thr, grad, hdr, st);
}

}  // namespace

bool span_backward_supported(int H, int W, int C) {
  return C >= 1 && C <= 16 && (long long)H * W * C < (1LL << 29);   // 32-bit frame offsets
}

hipError_t launch_backward_span(const float *params, const void *grad_image, float *grad_params,
                                int B, int N, int H, int W, int C, float radius, void *ws,
                                const Layout &L, bool check_stamp, hipStream_t st, int fmt) {
  char *w = (char *)ws;
  WsHeader *hdr = (WsHeader *)(w + L.hdr);
  const GRec *recs = (const GRec *)(w + L.recs);
  const ThinRec *thin = (const ThinRec *)(w + L.thin);
  // stamp check only (nothing to zero: every gradient row is stored once)
  PDR_TIMED(PDR_K_ZERO, st,
            hipLaunchKernelGGL(k_span_stamp, dim3(1), dim3(64), 0, st, hdr, check_stamp ? 1 : 0, B,
                               N, H, W, C, radius, (unsigned long long)(uintptr_t)params));
  const float thr = (float)((double)radius * (double)radius * kKappa2);
  if (C <= 1) launch_span_cp<1>(recs, thin, params, grad_image, fmt, B, N, H, W, C, thr, grad_params, hdr, st);
  else if (C == 2) launch_span_cp<2>(recs, thin, params, grad_image, fmt, B, N, H, W, C, thr, grad_params, hdr, st);
  else if (C == 3) launch_span_cp<3>(recs, thin, params, grad_image, fmt, B, N, H, W, C, thr, grad_params, hdr, st);
  else if (C == 4) launch_span_cp<4>(recs, thin, params, grad_image, fmt, B, N, H, W, C, thr, grad_params, hdr, st);
  else if (C <= 8) launch_span_cp<8>(recs, thin, params, grad_image, fmt, B, N, H, W, C, thr, grad_params, hdr, st);
  else launch_span_cp<16>(recs, thin, params, grad_image, fmt, B, N, H, W, C, thr, grad_params, hdr, st);
  return hipGetLastError();
}

}  // namespace pdr
