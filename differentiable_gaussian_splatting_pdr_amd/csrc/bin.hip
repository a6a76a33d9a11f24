// bin.hip -- per-Gaussian preprocessing and tile binning.
//
//  k_preprocess   one thread per Gaussian: validity, fp64 pixel bounding box
//                 of the truncated ellipse q <= k^2, whitening rows.
//  k_bin<false>   per (frame, tile group): per-tile overlap counts.
//  k_scan         one workgroup: exclusive scan of the counts (wave64 DPP
//                 scan) -> tile offsets, pair total, overflow flag.
//  k_bin<true>    per (frame, tile group): the per-tile lists, ascending
//                 Gaussian index, at the scanned offsets.
//
// A tile group holds a rectangle of tiles and walks the frame's Gaussians in
// chunks; for each chunk it builds an LDS bit matrix [tile][Gaussian] of box
// overlaps and compacts every tile's bit row with a wave scan.  The lists are
// thus produced in ascending order with no sort and no global atomics.
#include "pdr_common.hpp"
#include "pdr_internal.hpp"

namespace pdr {

// The truncated ellipse's pixel box (x0..x1, y0..y1 inclusive, clamped to the
// image), computed in fp64 with no FMA contraction so that the box -- and so
// the tile lists -- are reproducible bit for bit:
//   ex = k sqrt((s1 c)^2 + (s2 s)^2), ey = k sqrt((s1 s)^2 + (s2 c)^2)
//   x0 = ceil(mx - ex - 1/2), x1 = floor(mx + ex - 1/2)
// A pixel x is inside iff its centre x + 1/2 lies in [mx - ex, mx + ex].
__device__ static void pixel_box(double mx, double my, double s1, double s2, double c, double s,
                                 double k, int H, int W, int *out) {
#pragma clang fp contract(off)
  double t1 = s1 * c, t2 = s2 * s;
  double t3 = s1 * s, t4 = s2 * c;
  double ex = k * sqrt(t1 * t1 + t2 * t2);
  double ey = k * sqrt(t3 * t3 + t4 * t4);
  double fx0 = ceil(mx - ex - 0.5), fx1 = floor(mx + ex - 0.5);
  double fy0 = ceil(my - ey - 0.5), fy1 = floor(my + ey - 0.5);
  fx0 = fmin(fmax(fx0, 0.0), (double)W);
  fx1 = fmin(fmax(fx1, -1.0), (double)(W - 1));
  fy0 = fmin(fmax(fy0, 0.0), (double)H);
  fy1 = fmin(fmax(fy1, -1.0), (double)(H - 1));
  out[0] = (int)fx0;
  out[1] = (int)fx1;
  out[2] = (int)fy0;
  out[3] = (int)fy1;
}

__device__ __forceinline__ float clamp_to_float(double v) {
  const double m = 3.4028234663852886e38;  // FLT_MAX
  return (float)fmin(fmax(v, -m), m);
}

__global__ __launch_bounds__(256) void k_preprocess(const float *__restrict__ params, int BN, int C,
                                                    int H, int W, float radius,
                                                    GRec *__restrict__ recs,
                                                    uint2 *__restrict__ boxes, WsHeader *hdr,
                                                    int stamp_N, unsigned long long stamp_ptr) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    hdr->stamp[0] = BN / stamp_N;
    hdr->stamp[1] = stamp_N;
    hdr->stamp[2] = H;
    hdr->stamp[3] = W;
    hdr->stamp[4] = C;
    hdr->stamp[5] = __float_as_int(radius);
    hdr->stamp[6] = (int)(unsigned)(stamp_ptr & 0xffffffffull);
    hdr->stamp[7] = (int)(unsigned)(stamp_ptr >> 32);
  }
  if (i >= BN) return;
  const float *g = params + (size_t)i * (5 + C);
  float mx = g[0], my = g[1], s1 = g[2], s2 = g[3], th = g[4];
  bool ok = isfinite(mx) && isfinite(my) && isfinite(s1) && isfinite(s2) && isfinite(th) &&
            s1 > 0.f && s2 > 0.f;
  for (int c = 0; c < C; ++c) ok = ok && isfinite(g[5 + c]);
  GRec r;
  r.mx = mx;
  r.my = my;
  r.l11 = r.l12 = r.l21 = r.l22 = 0.f;
  r.bx = kEmptyBox;
  r.by = kEmptyBox;
  if (ok) {
    double sn, cs;
    sincos((double)th, &sn, &cs);
    int b[4];
    pixel_box(mx, my, s1, s2, cs, sn, (double)radius, H, W, b);
    if (b[0] <= b[1] && b[2] <= b[3]) {
      r.bx = (unsigned)b[0] | ((unsigned)b[1] << 16);
      r.by = (unsigned)b[2] | ((unsigned)b[3] << 16);
    }
    double i1 = kKappa / (double)s1, i2 = kKappa / (double)s2;
    r.l11 = clamp_to_float(cs * i1);
    r.l12 = clamp_to_float(sn * i1);
    r.l21 = clamp_to_float(-sn * i2);
    r.l22 = clamp_to_float(cs * i2);
  }
  recs[i] = r;
  boxes[i] = make_uint2(r.bx, r.by);
}

// LDS bit matrix binning.  Grid: (groups per frame, B); 256 threads.
// Dynamic LDS: Tg * (NC / 32) words, NC a multiple of 64.
template <bool WRITE>
__global__ __launch_bounds__(kBinThreads) void k_bin(const uint2 *__restrict__ boxes, int N,
                                                     int nTx, int nTy, int gw, int gh, int ngx,
                                                     int NC, int *__restrict__ counts,
                                                     const int *__restrict__ tile_off,
                                                     int *__restrict__ list, const WsHeader *hdr) {
  extern __shared__ unsigned int bits[];
  __shared__ int base[kMaxGroupTiles];
  const int b = blockIdx.y;
  const int gx = blockIdx.x % ngx, gy = blockIdx.x / ngx;
  const int tx0 = gx * gw, ty0 = gy * gh;
  const int aw = min(gw, nTx - tx0), ah = min(gh, nTy - ty0);
  const int Tg = aw * ah;
  const int nT = nTx * nTy;
  const int words = NC >> 5;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (WRITE && (hdr->status & kStatusOverflow)) return;
  for (int lt = tid; lt < Tg; lt += kBinThreads) {
    int t = (ty0 + lt / aw) * nTx + tx0 + lt % aw;
    base[lt] = WRITE ? tile_off[(size_t)b * nT + t] : 0;
  }
  const uint2 *fb = boxes + (size_t)b * N;
  for (int c0 = 0; c0 < N; c0 += NC) {
    for (int w = tid; w < Tg * words; w += kBinThreads) bits[w] = 0u;
    __syncthreads();
    const int cn = min(NC, N - c0);
    for (int i = tid; i < cn; i += kBinThreads) {
      uint2 bx = fb[c0 + i];
      int x0 = (int)(bx.x & 0xffffu), x1 = (int)(bx.x >> 16);
      int y0 = (int)(bx.y & 0xffffu), y1 = (int)(bx.y >> 16);
      if (x0 > x1) continue;
      int ux0 = max(x0 / kTile, tx0), ux1 = min(x1 / kTile, tx0 + aw - 1);
      int uy0 = max(y0 / kTile, ty0), uy1 = min(y1 / kTile, ty0 + ah - 1);
      const unsigned int bit = 1u << (i & 31);
      const int wi = i >> 5;
      for (int ty = uy0; ty <= uy1; ++ty)
        for (int tx = ux0; tx <= ux1; ++tx)
          atomicOr(&bits[((ty - ty0) * aw + (tx - tx0)) * words + wi], bit);
    }
    __syncthreads();
    // compaction: a wave owns tiles wave, wave + 4, ...
    for (int lt = wave; lt < Tg; lt += kBinThreads / kWave) {
      int run = base[lt];
      const unsigned int *row = bits + (size_t)lt * words;
      for (int seg = 0; seg < words; seg += 2 * kWave) {
        int w0 = seg + 2 * lane;
        unsigned long long m = 0ull;
        if (w0 < words) m = (unsigned long long)row[w0] | ((unsigned long long)row[w0 + 1] << 32);
        int cnt = __popcll(m);
        int incl = wave_incl_scan(cnt);
        if (WRITE) {
          int pos = run + incl - cnt;
          int nb = c0 + w0 * 32;
          while (m) {
            int k = __ffsll((long long)m) - 1;
            list[pos++] = nb + k;
            m &= m - 1ull;
          }
        }
        run += wave_read(incl, 63);
      }
      if (lane == 0) base[lt] = run;
    }
    __syncthreads();
  }
  if (!WRITE) {
    for (int lt = tid; lt < Tg; lt += kBinThreads) {
      int t = (ty0 + lt / aw) * nTx + tx0 + lt % aw;
      counts[(size_t)b * nT + t] = base[lt];
    }
  }
}

// Exclusive scan of M int32 counts by one 1024-thread workgroup, 4096
// counts per step: thread-serial over 4, wave64 DPP scan, the 16 wave
// totals and the running carry combined in 64 bits by one thread.
__global__ __launch_bounds__(kScanThreads) void k_scan(const int *__restrict__ counts, long long M,
                                                       int *__restrict__ tile_off, long long cap,
                                                       WsHeader *hdr) {
  __shared__ long long wsum[kScanThreads / kWave];
  __shared__ long long carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (long long base = 0; base < M; base += 4 * kScanThreads) {
    long long idx = base + 4LL * tid;
    int v[4];
    for (int j = 0; j < 4; ++j) v[j] = (idx + j < M) ? counts[idx + j] : 0;
    int tsum = v[0] + v[1] + v[2] + v[3];
    int incl = wave_incl_scan(tsum);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    if (tid == 0) {
      // 16 wave totals: a serial exclusive scan in one lane, exact in 64 bits
      long long run = carry_s;
      for (int w = 0; w < kScanThreads / kWave; ++w) {
        long long t = wsum[w];
        wsum[w] = run;
        run += t;
      }
      carry_s = run;
    }
    __syncthreads();
    long long off = wsum[wave] + (incl - tsum);
    for (int j = 0; j < 4; ++j) {
      if (idx + j < M) tile_off[idx + j] = (int)off;
      off += v[j];
    }
    __syncthreads();
  }
  if (tid == 0) {
    long long tot = carry_s;
    tile_off[M] = (int)(tot > 0x7fffffffLL ? 0x7fffffffLL : tot);
    hdr->total = tot;
    hdr->cap = cap;
    // a fresh binning: clears any earlier overflow or stale flag
    int st = 0;
    if (tot > cap || tot > 0x7fffffffLL) st |= kStatusOverflow;
    hdr->status = st;
  }
}

// ----------------------------------------------------------------------------
// host launchers

static void choose_groups(int N, int nTx, int nTy, int *gw, int *gh, int *NC) {
  long long nc = ((long long)N + 63) / 64 * 64;
  if (nc > kMaxChunk) nc = kMaxChunk;
  *NC = (int)nc;
  int tmax = (int)((kBinLdsBytes * 8LL) / nc);  // tiles whose bit rows fit the LDS budget
  if (tmax > kMaxGroupTiles) tmax = kMaxGroupTiles;
  if (nTx * nTy <= tmax) {
    *gw = nTx;
    *gh = nTy;
  } else if (nTx <= tmax) {
    *gw = nTx;
    *gh = tmax / nTx;
  } else {
    *gw = tmax;
    *gh = 1;
  }
}

hipError_t launch_binning(const float *params, int B, int N, int H, int W, int C, float radius,
                          void *ws, const Layout &L, int *tile_off, int *list, long long cap,
                          bool stamp_valid, hipStream_t st) {
  char *w = (char *)ws;
  WsHeader *hdr = (WsHeader *)(w + L.hdr);
  GRec *recs = (GRec *)(w + L.recs);
  uint2 *boxes = (uint2 *)(w + L.boxes);
  int *counts = (int *)(w + L.counts);
  long long BN = (long long)B * N;
  int nTx = (W + kTile - 1) / kTile, nTy = (H + kTile - 1) / kTile;
  PDR_TIMED(PDR_K_PREPROCESS, st,
            hipLaunchKernelGGL(k_preprocess, dim3((unsigned)((BN + 255) / 256)), dim3(256), 0, st,
                               params, (int)BN, C, H, W, radius, recs, boxes, hdr, N,
                               stamp_valid ? (unsigned long long)(uintptr_t)params : 0ull));
  int gw, gh, NC;
  choose_groups(N, nTx, nTy, &gw, &gh, &NC);
  int ngx = (nTx + gw - 1) / gw, ngy = (nTy + gh - 1) / gh;
  size_t lds = (size_t)gw * gh * (NC / 32) * 4;
  dim3 grid((unsigned)(ngx * ngy), (unsigned)B);
  PDR_TIMED(PDR_K_BIN_COUNT, st,
            hipLaunchKernelGGL(k_bin<false>, grid, dim3(kBinThreads), lds, st, boxes, N, nTx, nTy,
                               gw, gh, ngx, NC, counts, (const int *)nullptr, (int *)nullptr,
                               (const WsHeader *)hdr));
  long long M = (long long)B * nTx * nTy;
  PDR_TIMED(PDR_K_SCAN, st,
            hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, st, (const int *)counts, M,
                               tile_off, cap, hdr));
  PDR_TIMED(PDR_K_BIN_WRITE, st,
            hipLaunchKernelGGL(k_bin<true>, grid, dim3(kBinThreads), lds, st, boxes, N, nTx, nTy,
                               gw, gh, ngx, NC, counts, (const int *)tile_off, list,
                               (const WsHeader *)hdr));
  return hipGetLastError();
}

}  // namespace pdr
