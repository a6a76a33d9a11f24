// raster.hip -- forward and backward tile rasterisation of the truncated
// anisotropic Gaussians, and the gradient finalisation.
//
// One wave64 workgroup per 16x16 tile.  Lane l owns the four pixels
// (x, y) = (l % 16, l / 16 + 4k), k = 0..3, of the tile, i.e. one pixel in
// each of four 16x4 strips.  The tile's Gaussian list is walked in batches of
// 64: each lane stages one Gaussian's record and amplitudes in LDS, then the
// wave reads them back one by one (broadcast).  Strips the Gaussian's pixel
// box misses are skipped with a scalar branch.
//
// Per (Gaussian, pixel): z = L (p - mu) with L the whitening rows scaled by
// sqrt(log2(e)/2), q' = z1^2 + z2^2, w = exp2(-q') if q' <= k^2 log2(e)/2.
// This equals exp(-q/2) with the Mahalanobis q of the definition.
//
// Forward: C channel accumulators per pixel in registers.
// Backward: per lane the partial sums over its pixels of
//   A_c = G_c w,  S1 = v z1, S2 = v z2, S11 = v z1^2, S22 = v z2^2, S12 = v z1 z2
// (v = w sum_c G_c a_c, z unscaled by 1/kappa), reduced across the wave by a
// transposed butterfly (each exchange halves the values a lane carries) so
// that after log2(K) steps every lane holds one sum; one global fp32 atomic
// per wave per Gaussian per sum then lands in grad_params, and a finalise
// kernel applies the chain rule in place.
#include "pdr_common.hpp"
#include "pdr_internal.hpp"

namespace pdr {

template <int CP>
struct BatchLds {
  GRec rec[kWave];
  float amp[kWave][CP];
  int idx[kWave];
};

template <int CP>
__device__ __forceinline__ void stage_batch(BatchLds<CP> &s, const GRec *__restrict__ recs,
                                            const float *__restrict__ params,
                                            const int *__restrict__ list, int s0, int cnt,
                                            size_t gbase, int P, int c0, int cc, int lane) {
  if (lane < cnt) {
    int n = list[s0 + lane];
    s.idx[lane] = n;
    s.rec[lane] = recs[gbase + n];
    const float *a = params + (gbase + n) * (size_t)P + 5 + c0;
#pragma unroll
    for (int c = 0; c < CP; ++c) s.amp[lane][c] = c < cc ? a[c] : 0.f;
  }
}

// strips k (rows ystrip0 + 4k .. + 3) met by the box rows [y0, y1]
__device__ __forceinline__ void strip_range(unsigned int by, int ystrip0, int *k0, int *k1) {
  int y0 = (int)(by & 0xffffu), y1 = (int)(by >> 16);
  *k0 = max(0, (y0 - ystrip0) >> 2);
  *k1 = min(3, (y1 - ystrip0) >> 2);
}

template <int CP>
__global__ __launch_bounds__(kWave) void k_forward(const GRec *__restrict__ recs,
                                                   const float *__restrict__ params,
                                                   const int *__restrict__ tile_off,
                                                   const int *__restrict__ list, int B, int N,
                                                   int H, int W, int C, int c0, int cc, float thr,
                                                   int nTx, int nT, float *__restrict__ image,
                                                   const WsHeader *hdr) {
  int f, t;
  if (!xcd_frame_item(blockIdx.x, nT, B, &f, &t)) return;
  if (hdr->status & kStatusOverflow) return;
  __shared__ BatchLds<CP> s;
  const int lane = threadIdx.x;
  const int tx = t % nTx, ty = t / nTx;
  const int px = tx * kTile + (lane & 15);
  const int py0 = ty * kTile + (lane >> 4);
  const int ystrip0 = ty * kTile;
  const float fx = (float)px + 0.5f, fy = (float)py0 + 0.5f;
  const int P = 5 + C;
  const size_t gbase = (size_t)f * N;
  float acc[4][CP];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int c = 0; c < CP; ++c) acc[k][c] = 0.f;

  const int beg = tile_off[(size_t)f * nT + t], end = tile_off[(size_t)f * nT + t + 1];
  for (int s0 = beg; s0 < end; s0 += kWave) {
    const int cnt = min(kWave, end - s0);
    __syncthreads();
    stage_batch<CP>(s, recs, params, list, s0, cnt, gbase, P, c0, cc, lane);
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const GRec r = s.rec[j];
      int k0, k1;
      strip_range(__builtin_amdgcn_readfirstlane(r.by), ystrip0, &k0, &k1);
      const float dx = fx - r.mx, dy = fy - r.my;
      const float z1 = r.l11 * dx + r.l12 * dy;
      const float z2 = r.l21 * dx + r.l22 * dy;
      const float st1 = 4.f * r.l12, st2 = 4.f * r.l22;
      float a[CP];
#pragma unroll
      for (int c = 0; c < CP; ++c) a[c] = s.amp[j][c];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < k0 || k > k1) continue;
        const float u1 = z1 + (float)k * st1;
        const float u2 = z2 + (float)k * st2;
        const float q = u1 * u1 + u2 * u2;
        const float w = q <= thr ? __builtin_amdgcn_exp2f(-q) : 0.f;
#pragma unroll
        for (int c = 0; c < CP; ++c) acc[k][c] += a[c] * w;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int py = py0 + 4 * k;
    if (px < W && py < H) {
      float *o = image + (((size_t)f * H + py) * W + px) * (size_t)C + c0;
#pragma unroll
      for (int c = 0; c < CP; ++c)
        if (c < cc) o[c] = acc[k][c];
    }
  }
}

// One exchange step of the transposed butterfly: lanes with (lane & MASK)
// keep the upper HALF values, the others the lower HALF, and add the
// partner's copy of the half they keep.
template <int HALF, int MASK>
__device__ __forceinline__ void tstep(float *v, bool up) {
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const float keep = up ? v[i + HALF] : v[i];
    const float send = up ? v[i] : v[i + HALF];
    v[i] = keep + xor_partner<MASK>(send);
  }
}

// Reduce KP per-lane values over the wave.  Afterwards every lane holds the
// wave total of value index bitrev_log2(KP)(lane & (KP - 1)).
template <int KP>
__device__ __forceinline__ float wave_reduce_transposed(float *v, int lane) {
  static_assert(KP == 8 || KP == 16 || KP == 32, "KP");
  tstep<KP / 2, 1>(v, lane & 1);
  tstep<KP / 4, 2>(v, lane & 2);
  tstep<KP / 8, 4>(v, lane & 4);
  if constexpr (KP >= 16) tstep<KP / 16, 8>(v, lane & 8);
  if constexpr (KP >= 32) tstep<KP / 32, 16>(v, lane & 16);
  float r = v[0];
  if constexpr (KP < 16) r = xor_sum<8>(r);
  if constexpr (KP < 32) r = xor_sum<16>(r);
  return xor_sum<32>(r);
}

template <int KP>
__device__ __forceinline__ int value_index(int lane) {
  int idx = 0;
#pragma unroll
  for (int s = 0, h = KP / 2; h >= 1; ++s, h >>= 1)
    if (lane & (1 << s)) idx += h;
  return idx;
}

template <int K>
struct Pow2Up {
  static constexpr int value = K <= 8 ? 8 : (K <= 16 ? 16 : 32);
};

template <int CP>
__global__ __launch_bounds__(kWave) void k_backward(const GRec *__restrict__ recs,
                                                    const float *__restrict__ params,
                                                    const float *__restrict__ gimg,
                                                    const int *__restrict__ tile_off,
                                                    const int *__restrict__ list, int B, int N,
                                                    int H, int W, int C, int c0, int cc,
                                                    float thr, int nTx, int nT,
                                                    float *__restrict__ sums, const WsHeader *hdr) {
  constexpr int K = CP + 5;
  constexpr int KP = Pow2Up<K>::value;
  int f, t;
  if (!xcd_frame_item(blockIdx.x, nT, B, &f, &t)) return;
  if (hdr->status & (kStatusOverflow | kStatusStale)) return;
  __shared__ BatchLds<CP> s;
  const int lane = threadIdx.x;
  const int tx = t % nTx, ty = t / nTx;
  const int px = tx * kTile + (lane & 15);
  const int py0 = ty * kTile + (lane >> 4);
  const int ystrip0 = ty * kTile;
  const float fx = (float)px + 0.5f, fy = (float)py0 + 0.5f;
  const int P = 5 + C;
  const size_t gbase = (size_t)f * N;

  float G[4][CP];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int py = py0 + 4 * k;
    const bool in = px < W && py < H;
    const float *g = gimg + (((size_t)f * H + (in ? py : 0)) * W + (in ? px : 0)) * (size_t)C + c0;
#pragma unroll
    for (int c = 0; c < CP; ++c) G[k][c] = (in && c < cc) ? g[c] : 0.f;
  }
  const int vidx = value_index<KP>(lane & (KP - 1));
  int slot = -1;
  if (lane < KP) {
    if (vidx < CP) slot = vidx < cc ? 5 + c0 + vidx : -1;
    else if (vidx < K) slot = vidx - CP;
  }

  const int beg = tile_off[(size_t)f * nT + t], end = tile_off[(size_t)f * nT + t + 1];
  for (int s0 = beg; s0 < end; s0 += kWave) {
    const int cnt = min(kWave, end - s0);
    __syncthreads();
    stage_batch<CP>(s, recs, params, list, s0, cnt, gbase, P, c0, cc, lane);
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const GRec r = s.rec[j];
      int k0, k1;
      strip_range(__builtin_amdgcn_readfirstlane(r.by), ystrip0, &k0, &k1);
      const float dx = fx - r.mx, dy = fy - r.my;
      const float z1 = r.l11 * dx + r.l12 * dy;
      const float z2 = r.l21 * dx + r.l22 * dy;
      const float st1 = 4.f * r.l12, st2 = 4.f * r.l22;
      float a[CP];
#pragma unroll
      for (int c = 0; c < CP; ++c) a[c] = s.amp[j][c];
      float part[KP];
#pragma unroll
      for (int i = 0; i < KP; ++i) part[i] = 0.f;
      bool any = false;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < k0 || k > k1) continue;
        const float u1 = z1 + (float)k * st1;
        const float u2 = z2 + (float)k * st2;
        const float q = u1 * u1 + u2 * u2;
        const bool inside = q <= thr;
        any = any || inside;
        const float w = inside ? __builtin_amdgcn_exp2f(-q) : 0.f;
        float h = 0.f;
#pragma unroll
        for (int c = 0; c < CP; ++c) h += G[k][c] * a[c];
        const float v = h * w;
#pragma unroll
        for (int c = 0; c < CP; ++c) part[c] += G[k][c] * w;
        const float t1 = v * u1, t2 = v * u2;
        part[CP + 0] += t1;
        part[CP + 1] += t2;
        part[CP + 2] += t1 * u1;
        part[CP + 3] += t2 * u2;
        part[CP + 4] += t1 * u2;
      }
      if (__builtin_amdgcn_ballot_w64(any) == 0ull) continue;
      const float tot = wave_reduce_transposed<KP>(part, lane);
      if (slot >= 0) unsafeAtomicAdd(sums + (gbase + s.idx[j]) * (size_t)P + slot, tot);
    }
  }
}

// grad_params holds the raw sums (S1, S2, S11, S22, S12, A_c) in its slots;
// apply the chain rule in place (fp64):
//   dmu = L^T (S1, S2) with L = [[c/s1, s/s1], [-s/s2, c/s2]],
//   ds1 = S11/s1, ds2 = S22/s2, dtheta = (s1/s2 - s2/s1) S12, da = A
// undoing the kappa scale of the whitened coordinates.
__global__ __launch_bounds__(256) void k_finalize(const float *__restrict__ params,
                                                  float *__restrict__ grad, long long BN, int C,
                                                  const WsHeader *hdr) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= BN) return;
  if (hdr->status & (kStatusOverflow | kStatusStale)) return;
  const int P = 5 + C;
  const float *g = params + i * P;
  float *o = grad + i * P;
  float mx = g[0], my = g[1], s1f = g[2], s2f = g[3], th = g[4];
  bool ok = isfinite(mx) && isfinite(my) && isfinite(s1f) && isfinite(s2f) && isfinite(th) &&
            s1f > 0.f && s2f > 0.f;
  for (int c = 0; c < C; ++c) ok = ok && isfinite(g[5 + c]);
  if (!ok) {
    for (int c = 0; c < P; ++c) o[c] = 0.f;
    return;
  }
  double sn, cs;
  sincos((double)th, &sn, &cs);
  const double s1 = s1f, s2 = s2f;
  const double S1 = o[0], S2 = o[1], S11 = o[2], S22 = o[3], S12 = o[4];
  o[0] = (float)(((cs / s1) * S1 - (sn / s2) * S2) / kKappa);
  o[1] = (float)(((sn / s1) * S1 + (cs / s2) * S2) / kKappa);
  o[2] = (float)(S11 / (kKappa2 * s1));
  o[3] = (float)(S22 / (kKappa2 * s2));
  o[4] = (float)(((s1 * s1 - s2 * s2) / (s1 * s2)) * S12 / kKappa2);
}

// Zero grad_params (the atomic targets) and, when the backward reuses the
// forward's binning, check the workspace stamp.
__global__ __launch_bounds__(256) void k_zero_verify(float *__restrict__ p, long long n,
                                                     WsHeader *hdr, int check, int B, int N, int H,
                                                     int W, int C, float radius,
                                                     unsigned long long ptr) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    int st = hdr->status & ~kStatusStale;
    if (check) {
      bool same = hdr->stamp[0] == B && hdr->stamp[1] == N && hdr->stamp[2] == H &&
                  hdr->stamp[3] == W && hdr->stamp[4] == C &&
                  hdr->stamp[5] == __float_as_int(radius) &&
                  hdr->stamp[6] == (int)(unsigned)(ptr & 0xffffffffull) &&
                  hdr->stamp[7] == (int)(unsigned)(ptr >> 32);
      if (!same) st |= kStatusStale;
    }
    hdr->status = st;
  }
  long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] = 0.f;
}

// ----------------------------------------------------------------------------
// host launchers

static int channel_pad(int cc) {
  if (cc <= 4) return cc;
  if (cc <= 8) return 8;
  return 16;
}

template <int CP>
static void launch_fwd_cp(dim3 grid, hipStream_t st, const GRec *recs, const float *params,
                          const int *tile_off, const int *list, int B, int N, int H, int W, int C,
                          int c0, int cc, float thr, int nTx, int nT, float *image,
                          const WsHeader *hdr) {
  PDR_TIMED(PDR_K_FORWARD_RASTER, st,
            hipLaunchKernelGGL(k_forward<CP>, grid, dim3(kWave), 0, st, recs, params, tile_off,
                               list, B, N, H, W, C, c0, cc, thr, nTx, nT, image, hdr));
}

template <int CP>
static void launch_bwd_cp(dim3 grid, hipStream_t st, const GRec *recs, const float *params,
                          const float *gimg, const int *tile_off, const int *list, int B, int N,
                          int H, int W, int C, int c0, int cc, float thr, int nTx, int nT,
                          float *sums, const WsHeader *hdr) {
  PDR_TIMED(PDR_K_BACKWARD_RASTER, st,
            hipLaunchKernelGGL(k_backward<CP>, grid, dim3(kWave), 0, st, recs, params, gimg,
                               tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, sums, hdr));
}

static float threshold(float radius) {
  // q' <= k^2 log2(e)/2, rounded once to fp32
  return (float)((double)radius * (double)radius * kKappa2);
}

hipError_t launch_forward_raster(const float *params, float *image, int B, int N, int H, int W,
                                 int C, float radius, void *ws, const Layout &L, hipStream_t st) {
  char *w = (char *)ws;
  const WsHeader *hdr = (const WsHeader *)(w + L.hdr);
  const GRec *recs = (const GRec *)(w + L.recs);
  const int *tile_off = (const int *)(w + L.tile_off);
  const int *list = (const int *)(w + L.list);
  int nTx = (W + kTile - 1) / kTile, nTy = (H + kTile - 1) / kTile, nT = nTx * nTy;
  dim3 grid((unsigned)xcd_grid(nT, B));
  float thr = threshold(radius);
  for (int c0 = 0; c0 < C; c0 += 16) {
    int cc = C - c0 < 16 ? C - c0 : 16;
    switch (channel_pad(cc)) {
      case 1: launch_fwd_cp<1>(grid, st, recs, params, tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, image, hdr); break;
      case 2: launch_fwd_cp<2>(grid, st, recs, params, tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, image, hdr); break;
      case 3: launch_fwd_cp<3>(grid, st, recs, params, tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, image, hdr); break;
      case 4: launch_fwd_cp<4>(grid, st, recs, params, tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, image, hdr); break;
      case 8: launch_fwd_cp<8>(grid, st, recs, params, tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, image, hdr); break;
      default: launch_fwd_cp<16>(grid, st, recs, params, tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, image, hdr); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_backward(const float *params, const float *grad_image, float *grad_params, int B,
                           int N, int H, int W, int C, float radius, void *ws, const Layout &L,
                           bool check_stamp, hipStream_t st) {
  char *w = (char *)ws;
  WsHeader *hdr = (WsHeader *)(w + L.hdr);
  const GRec *recs = (const GRec *)(w + L.recs);
  const int *tile_off = (const int *)(w + L.tile_off);
  const int *list = (const int *)(w + L.list);
  int nTx = (W + kTile - 1) / kTile, nTy = (H + kTile - 1) / kTile, nT = nTx * nTy;
  long long BN = (long long)B * N, total = BN * (5 + C);
  long long zb = (total + 255) / 256;
  if (zb > 8192) zb = 8192;
  PDR_TIMED(PDR_K_ZERO, st,
            hipLaunchKernelGGL(k_zero_verify, dim3((unsigned)zb), dim3(256), 0, st, grad_params,
                               total, hdr, check_stamp ? 1 : 0, B, N, H, W, C, radius,
                               (unsigned long long)(uintptr_t)params));
  dim3 grid((unsigned)xcd_grid(nT, B));
  float thr = threshold(radius);
  for (int c0 = 0; c0 < C; c0 += 16) {
    int cc = C - c0 < 16 ? C - c0 : 16;
    switch (channel_pad(cc)) {
      case 1: launch_bwd_cp<1>(grid, st, recs, params, grad_image, tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, grad_params, hdr); break;
      case 2: launch_bwd_cp<2>(grid, st, recs, params, grad_image, tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, grad_params, hdr); break;
      case 3: launch_bwd_cp<3>(grid, st, recs, params, grad_image, tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, grad_params, hdr); break;
      case 4: launch_bwd_cp<4>(grid, st, recs, params, grad_image, tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, grad_params, hdr); break;
      case 8: launch_bwd_cp<8>(grid, st, recs, params, grad_image, tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, grad_params, hdr); break;
      default: launch_bwd_cp<16>(grid, st, recs, params, grad_image, tile_off, list, B, N, H, W, C, c0, cc, thr, nTx, nT, grad_params, hdr); break;
    }
  }
  PDR_TIMED(PDR_K_FINALIZE, st,
            hipLaunchKernelGGL(k_finalize, dim3((unsigned)((BN + 255) / 256)), dim3(256), 0, st,
                               params, grad_params, BN, C, (const WsHeader *)hdr));
  return hipGetLastError();
}

}  // namespace pdr
