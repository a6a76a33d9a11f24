// raster.hip -- forward and backward tile rasterisation of the truncated
// anisotropic Gaussians, and the gradient finalisation.
//
// A 16x16 tile is covered by units of 64 pixels, UW x UH with UW * UH = 64
// (16x4 strips or 8x8 quads).  A wave64 owns UX x UY units (a region of
// UX*UW x UY*UH pixels); lane l owns pixel (l % UW, l / UW) of every one of
// its units, so a lane holds UX*UY pixels.  The waves of a workgroup cover
// the tile and share one LDS staging area: batches of
// the tile's Gaussian list (record + amplitudes) are loaded cooperatively,
// then every wave reads them back one by one (broadcast).  For each Gaussian
// a wave skips, with scalar branches, its units that the Gaussian's pixel
// box misses or that its truncated ellipse provably misses (decided once per
// entry at staging).
//
// Per (Gaussian, pixel): z = L (p - mu) with L the whitening rows scaled by
// sqrt(log2(e)/2), q' = z1^2 + z2^2, w = exp2(-q') if q' <= k^2 log2(e)/2.
// This equals exp(-q/2) with the Mahalanobis q of the definition.  p - mu
// is formed for every unit from exact tile-local coordinates (stepping z by
// whole units instead, z + 8 L e_x, loses eps |L| 16 to cancellation, which
// is visible for tiny Gaussians whose |L| ~ 1/s is large).
//
// Forward: C channel accumulators per pixel in registers.
// Backward: per lane the partial sums over its pixels of
//   A_c = G_c w,  S1 = v z1, S2 = v z2, S11 = v z1^2, S22 = v z2^2, S12 = v z1 z2
// (v = w sum_c G_c a_c, z in the scaled coordinates); a unit whose pixels
// all fall outside the truncation is skipped after the compare (wave
// ballot).  The sums are reduced across the wave by a transposed butterfly
// (each exchange halves the values a lane carries) so that after log2(K)
// steps every lane holds one total; one global fp32 atomic per wave per
// Gaussian per sum lands in grad_params, and a finalise kernel applies the
// chain rule in place.
#include <type_traits>

#include "pdr_common.hpp"
#include "pdr_internal.hpp"

namespace pdr {

template <int V>
using IC = std::integral_constant<int, V>;

template <int UW, int UX, int UY>
struct WaveLayout {
  static constexpr int kUH = kWave / UW;
  static constexpr int kRW = UX * UW, kRH = UY * kUH;  // wave region
  static_assert(kRW == kTileW && kTileH % kRH == 0, "a wave spans the tile's width");
  static constexpr int kWaves = kTileH / kRH;
  static constexpr int kUnitsPerWave = UX * UY;  // consecutive bits of the tile's unit mask
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kBatch = kThreads;  // list entries staged per round
};

// One staged list entry (interleaved so that a wave reads it from one LDS
// base address): the whitening rows, the mean relative to the tile origin
// (so that p - mu is formed from small tile-local numbers: exact for pixels
// near the mean; folding mu into an offset c = -L mu instead cancels
// catastrophically for tiny Gaussians, whose L is large), the mask of tile
// units the truncated ellipse may meet, the element offset of the Gaussian's
// parameter row, and its amplitudes.
template <int CP>
struct alignas(16) Entry {
  float l11, l12, l21, l22;
  float mx, my;
  unsigned int mask;
  int row;  // (frame * N + n) * (5 + C)
  float amp[(CP + 3) / 4 * 4];
};

// Conservative test that no pixel centre of a unit lies inside the
// truncated ellipse, as the rasters decide it.  With d = p - mu ranging over
// the rectangle [X0, X1] x [Y0, Y1] of the unit's pixel centres,
// q'(d) = |L d|^2 = A dx^2 + 2 Bc dx dy + Cc dy^2 is convex, so its minimum
// over the rectangle is 0 if the rectangle holds d = 0 and otherwise lies on
// an edge, where it is the clamped minimum of a 1-D quadratic (iA = 1/A,
// iC = 1/Cc).  An inexact minimiser only raises q' to second order; the unit
// is dropped only if the minimum exceeds thr by a margin of 1e-4 (thr + m2),
// m2 = ((|l11| + |l12|)^2 + (|l21| + |l22|)^2) max|d|^2 bounding the squared
// magnitudes of the terms, which covers the fp32 rounding here and in the
// rasters' own q' (a few ulp of those terms).
struct EllipseRows {
  float l11, l12, l21, l22, A, Bc, Cc, iA, iC, r2;
};
__device__ __forceinline__ bool unit_missed(const EllipseRows &E, float X0, float X1, float Y0,
                                            float Y1, float thr) {
  if (X0 <= 0.f && X1 >= 0.f && Y0 <= 0.f && Y1 >= 0.f) return false;
  auto qat = [&](float x, float y) { return (E.A * x) * x + (2.f * E.Bc * x) * y + (E.Cc * y) * y; };
  // edges y = Y0, Y1 (minimise over x), then x = X0, X1 (over y)
  const float xa = fminf(fmaxf(-E.Bc * Y0 * E.iA, X0), X1);
  const float xb = fminf(fmaxf(-E.Bc * Y1 * E.iA, X0), X1);
  const float ya = fminf(fmaxf(-E.Bc * X0 * E.iC, Y0), Y1);
  const float yb = fminf(fmaxf(-E.Bc * X1 * E.iC, Y0), Y1);
  const float qmin = fminf(fminf(qat(xa, Y0), qat(xb, Y1)), fminf(qat(X0, ya), qat(X1, yb)));
  const float dm = fmaxf(fmaxf(fabsf(X0), fabsf(X1)), fmaxf(fabsf(Y0), fabsf(Y1)));
  return qmin > thr + 1e-4f * (thr + E.r2 * dm * dm);
}

// Flag above the unit bits of a thin entry's mask: its rows were swapped
// for the compensated evaluation (the sums of the two rows trade places).
constexpr unsigned int kEntrySwap = 0x40000000u;

// Stages the list entries [s0, s0 + cnt) of the tile, one per thread of the
// workgroup (computed here, in parallel, so that the per-entry loop only
// reads and tests bits).  The unit mask holds the units the pixel box meets,
// less those the truncated ellipse misses.  A thin Gaussian's entry gets the
// split tile-local mean, its rows in thin-row-last order and, in sx at the
// same slot, the compensation constants (the forward rasters, FWD, take it
// above a higher anisotropy than the backward).  Plain entries are written first
// and thin ones after them, each group in list order, so that the rasters
// run one loop per evaluation with no per-entry branch between them; the
// number of plain entries is returned (wave-uniform).  scnt: 2 * WAVES
// ints of LDS (used with more than one wave).
template <int CP, int UW, int WAVES, bool FWD>
__device__ __forceinline__ int stage_batch(Entry<CP> *s, ThinX *sx, int *scnt,
                                           const GRec *__restrict__ recs,
                                           const ThinRec *__restrict__ thin,
                                           const float *__restrict__ params,
                                           const int *__restrict__ list, int s0, int cnt,
                                           size_t gbase, int P, int c0, int cc, int tid, int tx0,
                                           int ty0, float thr) {
  constexpr int UH = kWave / UW, NUX = kTileW / UW, NUY = kTileH / UH;
  Entry<CP> e;
  ThinX tx{};
  bool is_thin_entry = false;
  if (tid < cnt) {
    const int n = list[s0 + tid];
    const GRec r = recs[gbase + n];
    e.l11 = r.l11;
    e.l12 = r.l12;
    e.l21 = r.l21;
    e.l22 = r.l22;
    e.mx = r.mx - (float)tx0;
    e.my = r.my - (float)ty0;
    e.row = ((int)gbase + n) * P;
    const float *a = params + (size_t)e.row + 5 + c0;
#pragma unroll
    for (int c = 0; c < (CP + 3) / 4 * 4; ++c) e.amp[c] = c < cc ? a[c] : 0.f;
    // listed => the box meets the tile; clamp it to the tile's units
    const int ux0 = max(0, ((int)(r.bx & 0xffffu) - tx0) / UW);
    const int ux1 = min(NUX - 1, ((int)(r.bx >> 16) - tx0) / UW);
    const int uy0 = max(0, ((int)(r.by & 0xffffu) - ty0) / UH);
    const int uy1 = min(NUY - 1, ((int)(r.by >> 16) - ty0) / UH);
    const unsigned int rowm = ((2u << ux1) - 1u) & ~((1u << ux0) - 1u);
    unsigned int m = 0u;
#pragma unroll
    for (int j = 0; j < NUY; ++j)
      if (j >= uy0 && j <= uy1) m |= rowm << (j * NUX);
    EllipseRows E;
    E.l11 = e.l11; E.l12 = e.l12; E.l21 = e.l21; E.l22 = e.l22;
    E.A = e.l11 * e.l11 + e.l21 * e.l21;
    E.Bc = e.l11 * e.l12 + e.l21 * e.l22;
    E.Cc = e.l12 * e.l12 + e.l22 * e.l22;
    E.iA = __builtin_amdgcn_rcpf(E.A);
    E.iC = __builtin_amdgcn_rcpf(E.Cc);
    const float r1 = fabsf(e.l11) + fabsf(e.l12), r2 = fabsf(e.l21) + fabsf(e.l22);
    E.r2 = r1 * r1 + r2 * r2;
    for (int u = 0; u < NUX * NUY; ++u) {
      if (!(m & (1u << u))) continue;
      const float X0 = (float)((u % NUX) * UW) + 0.5f - e.mx;
      const float Y0 = (float)((u / NUX) * UH) + 0.5f - e.my;
      if (unit_missed(E, X0, X0 + (float)(UW - 1), Y0, Y0 + (float)(UH - 1), thr))
        m &= ~(1u << u);
    }
    if (is_thin(e.l11, e.l12, e.l21, e.l22, FWD ? kThinRatio2Fwd : kThinRatio2)) {
      const ThinRec tr = thin[gbase + n];
      if (tr.flags & kThinOk) {
        is_thin_entry = true;
        if (tr.flags & kThinSwap) {
          float f = e.l11; e.l11 = e.l21; e.l21 = f;
          f = e.l12; e.l12 = e.l22; e.l22 = f;
          m |= kEntrySwap;
        }
        e.mx = tr.mhx - (float)tx0;   // exact: multiples of 2^-8 below 2^16
        e.my = tr.mhy - (float)ty0;
        tx = ThinX{tr.lo21, tr.lo22, tr.c1, tr.c2};
      }
    }
    e.mask = m;
  }
  // slots: plain entries first, then thin ones, list order within each
  const unsigned long long tb = __builtin_amdgcn_ballot_w64(tid < cnt && is_thin_entry);
  const unsigned long long pb = __builtin_amdgcn_ballot_w64(tid < cnt && !is_thin_entry);
  const int below_t = __builtin_amdgcn_mbcnt_hi((unsigned)(tb >> 32),
                                                __builtin_amdgcn_mbcnt_lo((unsigned)tb, 0u));
  const int below_p = __builtin_amdgcn_mbcnt_hi((unsigned)(pb >> 32),
                                                __builtin_amdgcn_mbcnt_lo((unsigned)pb, 0u));
  int nplain, pos;
  if constexpr (WAVES == 1) {
    nplain = __popcll(pb);
    pos = is_thin_entry ? nplain + below_t : below_p;
  } else {
    const int wave = tid >> 6;
    if ((tid & 63) == 0) {
      scnt[wave] = __popcll(pb);
      scnt[WAVES + wave] = __popcll(tb);
    }
    __syncthreads();
    int pbefore = 0, tbefore = 0;
    nplain = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      pbefore += w < wave ? scnt[w] : 0;
      tbefore += w < wave ? scnt[WAVES + w] : 0;
      nplain += scnt[w];
    }
    pos = is_thin_entry ? nplain + tbefore + below_t : pbefore + below_p;
    nplain = __builtin_amdgcn_readfirstlane(nplain);
  }
  if (tid < cnt) {
    s[pos] = e;
    if (is_thin_entry) sx[pos] = tx;
  }
  return nplain;
}

// The compensation constants of an entry in scalar registers (they are
// wave-uniform; the thin loops then hold no more vector registers than the
// plain ones).
__device__ __forceinline__ float sgpr(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
__device__ __forceinline__ ThinX uniform(const ThinX &t) {
  return ThinX{sgpr(t.lo21), sgpr(t.lo22), sgpr(t.c1), sgpr(t.c2)};
}

// Where the image (forward output, backward input) lives: value (pixel, c)
// at pixel * ldo + ooff + c.  With concat fusion (ldo = Cp + C, ooff = Cp)
// the first Cp channels of every pixel belong to the pixel branch: the
// forward copies them from xin, the backward copies their gradient to xout.
// fmt selects the image's storage: fp32, or fp16 / bf16 (round to nearest
// even from the fp32 accumulators; fp32 arithmetic throughout).
struct ImgView {
  int ldo, ooff;
  const float *xin;
  float *xout;
  int Cp;
  int fmt;
};

__device__ __forceinline__ void store_image(void *base, size_t idx, float v, int fmt) {
  if (fmt == PDR_FMT_F32) {
    static_cast<float *>(base)[idx] = v;
  } else if (fmt == PDR_FMT_F16) {
    static_cast<_Float16 *>(base)[idx] = (_Float16)v;
  } else {
    static_cast<__bf16 *>(base)[idx] = (__bf16)v;
  }
}

__device__ __forceinline__ float load_image(const void *base, size_t idx, int fmt) {
  if (fmt == PDR_FMT_F32) return static_cast<const float *>(base)[idx];
  if (fmt == PDR_FMT_F16) return (float)static_cast<const _Float16 *>(base)[idx];
  return (float)static_cast<const __bf16 *>(base)[idx];
}

// Orders one wave's LDS accesses across its lanes (a wave's LDS operations
// execute in order; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// FS > 1 (one-wave tile layouts only): FS waves per tile, each walking a
// contiguous share of the tile's list with its own staging area and no
// workgroup barrier, their per-pixel sums added in wave order at the end
// (deterministic).  For batches of few tiles, where one wave per tile
// leaves the SIMDs short of resident waves.
template <int CP, int UW, int UX, int UY, int FS = 1>
__global__ __launch_bounds__((WaveLayout<UW, UX, UY>::kThreads * FS)) void k_forward(
    const GRec *__restrict__ recs, const ThinRec *__restrict__ thin,
    const float *__restrict__ params, const int *__restrict__ tile_off,
    const int *__restrict__ list, int B, int N, int H, int W, int C, int c0, int cc, float thr,
    int nTx, int nT, void *__restrict__ image, ImgView iv,
    const WsHeader *hdr, const int *__restrict__ order) {
  using WL = WaveLayout<UW, UX, UY>;
  static_assert(FS == 1 || WL::kWaves == 1, "list shares need a one-wave tile layout");
  constexpr int UH = WL::kUH;
  int f, t;
  // Lists that overflowed are incomplete, and so is the tile order: every
  // pixel of such a call is set to NaN, tiles taken in launch order.
  const bool ovf = (hdr->status & kStatusOverflow) != 0;
  if ((order && !ovf) ? !ordered_tile(blockIdx.x, nT, B, order, &f, &t)
                      : !xcd_frame_item(blockIdx.x, nT, B, &f, &t))
    return;
  __shared__ Entry<CP> s_all[FS][WL::kBatch];
  __shared__ ThinX sx_all[FS][WL::kBatch];
  __shared__ int scnt[2 * WL::kWaves];
  const int tid = threadIdx.x, lane = tid & 63;
  // region wave (tile layouts of several waves) and list share (FS > 1)
  const int wave = FS > 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6);
  const int part = FS > 1 ? __builtin_amdgcn_readfirstlane(tid >> 6) : 0;
  const int stid = FS > 1 ? lane : tid;   // thread index within the staging group
  Entry<CP> *s = s_all[part];
  ThinX *sx = sx_all[part];
  const int tx0 = (t % nTx) * kTileW, ty0 = (t / nTx) * kTileH;
  const int rx0 = tx0, ry0 = ty0 + wave * WL::kRH;
  const int mshift = wave * WL::kUnitsPerWave;
  const int lx = lane % UW, ly = lane / UW;
  // tile-local pixel centre of the lane in its first unit
  const float fx = (float)(rx0 - tx0 + lx) + 0.5f, fy = (float)(ry0 - ty0 + ly) + 0.5f;
  const int P = 5 + C;
  const size_t gbase = (size_t)f * N;
  float acc[UY][UX][CP];
#pragma unroll
  for (int j = 0; j < UY; ++j)
#pragma unroll
    for (int i = 0; i < UX; ++i)
#pragma unroll
      for (int c = 0; c < CP; ++c) acc[j][i][c] = ovf ? __builtin_nanf("") : 0.f;

  int beg = 0, end = 0;
  if (!ovf) {
    beg = __builtin_amdgcn_readfirstlane(tile_off[(size_t)f * nT + t]);
    end = __builtin_amdgcn_readfirstlane(tile_off[(size_t)f * nT + t + 1]);
  }
  if constexpr (FS > 1) {
    const int share = (end - beg + FS - 1) / FS;
    beg = min(end, beg + part * share);
    end = min(end, beg + share);
  }
  for (int s0 = beg; s0 < end; s0 += WL::kBatch) {
    const int cnt = min(WL::kBatch, end - s0);
    if constexpr (FS > 1) wave_lds_sync(); else __syncthreads();
    const int np = stage_batch<CP, UW, WL::kWaves, true>(s, sx, scnt, recs, thin, params, list, s0, cnt,
                                                   gbase, P, c0, cc, stid, tx0, ty0, thr);
    if constexpr (FS > 1) wave_lds_sync(); else __syncthreads();
    // the entry loops run on scalar counts; each entry is read whole (its
    // unit mask is all but never empty for a listed Gaussian).  THIN: the
    // compensated evaluation of the batch's thin entries, after the others.
    auto run = [&](auto thinc, int e0, int e1) {
      constexpr bool THIN = decltype(thinc)::value != 0;
      for (int e = e0; e < e1; ++e) {
        const Entry<CP> r = s[e];
        const unsigned int um =
            (__builtin_amdgcn_readfirstlane(r.mask) >> mshift) & ((1u << WL::kUnitsPerWave) - 1u);
        if (um == 0u) continue;
        ThinX tx{};
        if constexpr (THIN) tx = uniform(sx[e]);
        float a[CP];
#pragma unroll
        for (int c = 0; c < CP; ++c) a[c] = r.amp[c];
#pragma unroll
        for (int j = 0; j < UY; ++j) {
          if (!(um & (((1u << UX) - 1u) << (j * UX)))) continue;
          const float dy = (fy + (float)(UH * j)) - r.my;
#pragma unroll
          for (int i = 0; i < UX; ++i) {
            if (!(um & (1u << (j * UX + i)))) continue;
            const float dx = (fx + (float)(UW * i)) - r.mx;
            float u1, u2;
            whiten<THIN>(r.l11, r.l12, r.l21, r.l22, tx, dx, dy, u1, u2);
            const float q = u1 * u1 + u2 * u2;
            const float w = q <= thr ? __builtin_amdgcn_exp2f(-q) : 0.f;
#pragma unroll
            for (int c = 0; c < CP; ++c) acc[j][i][c] += a[c] * w;
          }
        }
      }
    };
    run(IC<0>{}, 0, np);
    run(IC<1>{}, np, __builtin_amdgcn_readfirstlane(cnt));
  }
  if constexpr (FS > 1) {   // the shares' sums, added in wave order by wave 0
    constexpr int V = UY * UX * CP;
    __shared__ float red[(FS - 1) * V * kWave];
    if (part > 0) {
#pragma unroll
      for (int j = 0; j < UY; ++j)
#pragma unroll
        for (int i = 0; i < UX; ++i)
#pragma unroll
          for (int c = 0; c < CP; ++c)
            red[((part - 1) * V + (j * UX + i) * CP + c) * kWave + lane] = acc[j][i][c];
    }
    __syncthreads();
    if (part > 0) return;
    for (int w = 1; w < FS; ++w) {
#pragma unroll
      for (int j = 0; j < UY; ++j)
#pragma unroll
        for (int i = 0; i < UX; ++i)
#pragma unroll
          for (int c = 0; c < CP; ++c)
            acc[j][i][c] += red[((w - 1) * V + (j * UX + i) * CP + c) * kWave + lane];
    }
  }
#pragma unroll
  for (int j = 0; j < UY; ++j) {
#pragma unroll
    for (int i = 0; i < UX; ++i) {
      const int px = rx0 + UW * i + lx, py = ry0 + UH * j + ly;
      if (px < W && py < H) {
        const size_t pix = ((size_t)f * H + py) * W + px;
        const size_t o = pix * (size_t)iv.ldo + iv.ooff + c0;
#pragma unroll
        for (int c = 0; c < CP; ++c)
          if (c < cc) store_image(image, o + c, acc[j][i][c], iv.fmt);
        if (iv.xin) {   // concat fusion: the pixel branch's channels go first
          const float *xi = iv.xin + pix * (size_t)iv.Cp;
          float *ob = static_cast<float *>(image) + pix * (size_t)iv.ldo;   // fp32 only
          for (int c = 0; c < iv.Cp; ++c) ob[c] = xi[c];
        }
      }
    }
  }
}

// Support count: the forward raster's traversal (same lists, staged unit
// masks and fp32 q' per unit) with the accumulation replaced by a count of
// the lanes inside the truncation whose pixel lies in the frame (a ragged
// tile's lanes past the frame edge are evaluated but never stored); one
// 64-bit atomic per wave.  The number of (Gaussian, pixel) pairs the
// forward accumulates into the image, used as the work count of throughput
// figures.
template <int UW, int UX, int UY>
__global__ __launch_bounds__((WaveLayout<UW, UX, UY>::kThreads)) void k_count_support(
    const GRec *__restrict__ recs, const ThinRec *__restrict__ thin,
    const float *__restrict__ params, const int *__restrict__ tile_off,
    const int *__restrict__ list, int B, int N, int H, int W, int C, float thr, int nTx, int nT,
    unsigned long long *__restrict__ count,
    const WsHeader *hdr) {
  using WL = WaveLayout<UW, UX, UY>;
  constexpr int UH = WL::kUH;
  int f, t;
  if (!xcd_frame_item(blockIdx.x, nT, B, &f, &t)) return;
  if (hdr->status & kStatusOverflow) return;
  __shared__ Entry<1> s[WL::kBatch];
  __shared__ ThinX sx[WL::kBatch];
  __shared__ int scnt[2 * WL::kWaves];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tx0 = (t % nTx) * kTileW, ty0 = (t / nTx) * kTileH;
  const int ry0 = ty0 + wave * WL::kRH;
  const int mshift = wave * WL::kUnitsPerWave;
  const int lx = lane % UW, ly = lane / UW;
  const float fx = (float)lx + 0.5f, fy = (float)(ry0 - ty0 + ly) + 0.5f;
  const int P = 5 + C;
  const size_t gbase = (size_t)f * N;
  unsigned long long n_in = 0;  // wave-uniform
  const int beg = __builtin_amdgcn_readfirstlane(tile_off[(size_t)f * nT + t]);
  const int end = __builtin_amdgcn_readfirstlane(tile_off[(size_t)f * nT + t + 1]);
  for (int s0 = beg; s0 < end; s0 += WL::kBatch) {
    const int cnt = min(WL::kBatch, end - s0);
    __syncthreads();
    const int np = stage_batch<1, UW, WL::kWaves, true>(s, sx, scnt, recs, thin, params, list, s0, cnt,
                                                  gbase, P, 0, 1, tid, tx0, ty0, thr);
    __syncthreads();
    auto run = [&](auto thinc, int e0, int e1) {
      constexpr bool THIN = decltype(thinc)::value != 0;
      for (int e = e0; e < e1; ++e) {
        const Entry<1> r = s[e];
        const unsigned int um =
            (__builtin_amdgcn_readfirstlane(r.mask) >> mshift) & ((1u << WL::kUnitsPerWave) - 1u);
        if (um == 0u) continue;
        ThinX tx{};
        if constexpr (THIN) tx = uniform(sx[e]);
#pragma unroll
        for (int j = 0; j < UY; ++j) {
          if (!(um & (((1u << UX) - 1u) << (j * UX)))) continue;
          const float dy = (fy + (float)(UH * j)) - r.my;
          const bool row_in = ry0 + UH * j + ly < H;
#pragma unroll
          for (int i = 0; i < UX; ++i) {
            if (!(um & (1u << (j * UX + i)))) continue;
            const float dx = (fx + (float)(UW * i)) - r.mx;
            float u1, u2;
            whiten<THIN>(r.l11, r.l12, r.l21, r.l22, tx, dx, dy, u1, u2);
            const float q = u1 * u1 + u2 * u2;
            const bool in_frame = row_in && tx0 + UW * i + lx < W;
            n_in += __popcll(__builtin_amdgcn_ballot_w64(q <= thr && in_frame));
          }
        }
      }
    };
    run(IC<0>{}, 0, np);
    run(IC<1>{}, np, __builtin_amdgcn_readfirstlane(cnt));
  }
  if (lane == 0 && n_in) atomicAdd(count, n_in);
}

__global__ void k_zero_count(unsigned long long *count) { *count = 0ull; }

// Wave reduction through an LDS transpose: every lane writes its K values
// value-major (row k of red, rows padded to 68 words so that the vector
// reads below spread over the banks); lane l = g * GL + m (GL = 64 / KP
// lanes per value) then adds the KP consecutive words red[g][m KP ..
// m KP + KP) with 16-byte reads, and the GL lanes of a group add up by DPP.
// Lane g GL ends with the wave total of value g (g < K; the lanes of rows
// K..KP-1 read words nobody wrote and are not used).  Each wave owns its
// rows; a wave's LDS operations execute in order, so no barrier is needed.
// Fewer VALU instructions than the transposed butterfly, but two LDS round
// trips per list entry: measured 8% faster for one channel (K = 6) and
// 4-6% slower from three channels up, so it serves CP == 1 only.
#ifndef PDR_XPOSE_ONE_CHANNEL
#define PDR_XPOSE_ONE_CHANNEL 1
#endif
template <int CP>
struct UseXpose {
  static constexpr bool value = CP == 1 && PDR_XPOSE_ONE_CHANNEL;
};
constexpr int kRedRow = kWave + 4;
template <int K, int KP>
__device__ __forceinline__ float wave_reduce_xpose(const float *v, float *red, int lane) {
  constexpr int GL = kWave / KP;
#pragma unroll
  for (int k = 0; k < K; ++k) red[k * kRedRow + lane] = v[k];
  const int g = lane / GL, m = lane % GL;
  const float4 *src = reinterpret_cast<const float4 *>(red + g * kRedRow + m * KP);
  float4 x = src[0];
  float r = (x.x + x.y) + (x.z + x.w);
#pragma unroll
  for (int q = 1; q < KP / 4; ++q) {
    x = src[q];
    r += (x.x + x.y) + (x.z + x.w);
  }
  if constexpr (GL >= 2) r += xor_partner<1>(r);
  if constexpr (GL >= 4) r += xor_partner<2>(r);
  if constexpr (GL >= 8) r += dpp_row_shl<4>(r);  // lane 8 g reads lane 8 g + 4
  return r;
}

// Calls fn(IC<u>, IC<1>) for the lowest unit u of the mask um (non-empty),
// then fn(IC<v>, IC<0>) for every later unit v in um, each with its index
// known at compile time.
template <int U, int NU, class Fn>
__device__ __forceinline__ void for_units_after(unsigned int um, Fn &fn) {
  if constexpr (U < NU) {
    if (um & (1u << U)) fn(IC<U>{}, IC<0>{});
    for_units_after<U + 1, NU>(um, fn);
  }
}
template <int NU, int F = 0, class Fn>
__device__ __forceinline__ void for_units_from_first(unsigned int um, Fn &fn) {
  if constexpr (F < NU - 1) {
    if (um & (1u << F)) {
      fn(IC<F>{}, IC<1>{});
      for_units_after<F + 1, NU>(um, fn);
    } else {
      for_units_from_first<NU, F + 1>(um, fn);
    }
  } else {
    fn(IC<F>{}, IC<1>{});
  }
}

template <int K>
struct Pow2Up {
  static constexpr int value = K <= 8 ? 8 : (K <= 16 ? 16 : 32);
};

template <int CP, int UW, int UX, int UY, bool SPLIT = false>
__global__ __launch_bounds__((WaveLayout<UW, UX, UY>::kThreads)) void k_backward(
    const GRec *__restrict__ recs, const ThinRec *__restrict__ thin,
    const float *__restrict__ params, const void *__restrict__ gimg,
    const int *__restrict__ tile_off,
    const int *__restrict__ list, int B, int N, int H, int W, int C, int c0, int cc, float thr,
    int nTx, int nT, float *__restrict__ sums, ImgView iv, WsHeader *hdr,
    const int *__restrict__ order, int splits) {
  using WL = WaveLayout<UW, UX, UY>;
  constexpr int UH = WL::kUH;
  constexpr int K = CP + 5;
  constexpr int KP = Pow2Up<K>::value;
  int f, t, part = 0;
  // SPLIT: a tile's list is walked by `splits` workgroups, each taking a
  // contiguous share of its entries (every entry's sums leave through
  // atomics, so the shares need no combining); a compile-time variant, so
  // that the one-workgroup kernel carries none of it
  int bid = (int)blockIdx.x;
  if constexpr (SPLIT) bid = split_block(blockIdx.x, splits, &part);
  if (hdr->status & (kStatusOverflow | kStatusStale)) {
    // Binning that overflowed, or lists that are not this call's: no lists
    // to walk.  The finalisation sets dL/dparams to NaN; the pixel branch's
    // gradient slice (concat) is set to NaN here, tiles in launch order.
    if (iv.xout && (!SPLIT || part == 0) && xcd_frame_item(bid, nT, B, &f, &t)) {
      const int px0 = (t % nTx) * kTileW, py0 = (t / nTx) * kTileH;
      for (int k = threadIdx.x; k < kTileW * kTileH; k += WL::kThreads) {
        const int px = px0 + k % kTileW, py = py0 + k / kTileW;
        if (px >= W || py >= H) continue;
        float *xo = iv.xout + (((size_t)f * H + py) * W + px) * (size_t)iv.Cp;
        for (int c = 0; c < iv.Cp; ++c) xo[c] = __builtin_nanf("");
      }
    }
    return;
  }
  if (order ? !ordered_tile(bid, nT, B, order, &f, &t) : !xcd_frame_item(bid, nT, B, &f, &t))
    return;
  __shared__ Entry<CP> s[WL::kBatch];
  __shared__ ThinX sx[WL::kBatch];
  __shared__ int scnt[2 * WL::kWaves];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int tx0 = (t % nTx) * kTileW, ty0 = (t / nTx) * kTileH;
  const int rx0 = tx0, ry0 = ty0 + wave * WL::kRH;
  const int mshift = wave * WL::kUnitsPerWave;
  const int lx = lane % UW, ly = lane / UW;
  // tile-local pixel centre of the lane in its first unit
  const float fx = (float)(rx0 - tx0 + lx) + 0.5f, fy = (float)(ry0 - ty0 + ly) + 0.5f;
  const int P = 5 + C;
  const size_t gbase = (size_t)f * N;

  float G[UY][UX][CP];
#pragma unroll
  for (int j = 0; j < UY; ++j) {
#pragma unroll
    for (int i = 0; i < UX; ++i) {
      const int px = rx0 + UW * i + lx, py = ry0 + UH * j + ly;
      const bool in = px < W && py < H;
      const size_t pix = ((size_t)f * H + (in ? py : 0)) * W + (in ? px : 0);
      const size_t g = pix * (size_t)iv.ldo + iv.ooff + c0;
#pragma unroll
      for (int c = 0; c < CP; ++c) G[j][i][c] = (in && c < cc) ? load_image(gimg, g + c, iv.fmt) : 0.f;
      if (iv.xout && in && (!SPLIT || part == 0)) {   // concat fusion: the pixel branch's gradient slice (fp32 only)
        const float *gb = static_cast<const float *>(gimg) + pix * (size_t)iv.ldo;
        float *xo = iv.xout + pix * (size_t)iv.Cp;
        for (int c = 0; c < iv.Cp; ++c) xo[c] = gb[c];
      }
    }
  }
  // Non-finite dL/dI.  The evaluation multiplies every lane's G by its
  // weight, and a lane outside the truncation (w = 0) would turn a NaN or an
  // infinity there into NaN.  So the raster takes non-finite values as 0 and
  // flags their presence in the workspace header; the finalisation then adds
  // the terms of those values on the pixels of each Gaussian's support, so
  // that a non-finite value reaches exactly the sums of the Gaussians whose
  // support holds its pixel.
  bool bad = false;
#pragma unroll
  for (int j = 0; j < UY; ++j)
#pragma unroll
    for (int i = 0; i < UX; ++i)
#pragma unroll
      for (int c = 0; c < CP; ++c) {
        const bool fin = __builtin_isfinite(G[j][i][c]);
        bad |= !fin;
        G[j][i][c] = fin ? G[j][i][c] : 0.f;
      }
  if (__builtin_amdgcn_ballot_w64(bad) && lane == 0) hdr->nonfinite = 1;
  // which value's wave total a lane holds after the reduction, and whether
  // it issues that value's atomic
  constexpr bool kXpose = UseXpose<CP>::value;
  __shared__ __align__(16) float red_all[kXpose ? WL::kWaves * KP * kRedRow : 1];
  float *red = red_all + (kXpose ? wave * KP * kRedRow : 0);  // this wave's rows
  // With 16 channels the 21 sums would fill a 32-value butterfly with 11
  // zeros; instead the amplitude sums take a 16-value one and the five
  // moments an 8-value one (53 instead of 70 VALU per entry, a second
  // atomic instruction).
  constexpr bool kSplit = CP == 16;
  const int vidx = kXpose ? lane / (kWave / KP) : value_index<kSplit ? 16 : KP>(lane);
  int slot = -1, slot_m = -1;
  if constexpr (kSplit) {
    if (reduce_issuer<16>(lane)) slot = vidx < cc ? 5 + c0 + vidx : -1;
    if (reduce_issuer<8>(lane) && value_index<8>(lane) < 5) slot_m = value_index<8>(lane);
  } else if (kXpose ? lane % (kWave / KP) == 0 : reduce_issuer<KP>(lane)) {
    if (vidx < CP) slot = vidx < cc ? 5 + c0 + vidx : -1;
    else if (vidx < K) slot = vidx - CP;
  }

  int beg = __builtin_amdgcn_readfirstlane(tile_off[(size_t)f * nT + t]);
  int end = __builtin_amdgcn_readfirstlane(tile_off[(size_t)f * nT + t + 1]);
  if constexpr (SPLIT) {
    const int share = (end - beg + splits - 1) / splits;
    beg = min(end, beg + part * share);
    end = min(end, beg + share);
  }
  for (int s0 = beg; s0 < end; s0 += WL::kBatch) {
    const int cnt = min(WL::kBatch, end - s0);
    __syncthreads();
    const int np = stage_batch<CP, UW, WL::kWaves, false>(s, sx, scnt, recs, thin, params, list, s0, cnt,
                                                   gbase, P, c0, cc, tid, tx0, ty0, thr);
    __syncthreads();
    // the entry loops run on scalar counts; each entry is read whole (its
    // unit mask is all but never empty for a listed Gaussian).  THIN: the
    // compensated evaluation of the batch's thin entries, after the others.
    auto run = [&](auto thinc, int e0, int e1) {
      constexpr bool THIN = decltype(thinc)::value != 0;
      for (int e = e0; e < e1; ++e) {
        const Entry<CP> r = s[e];
        const unsigned int fl = __builtin_amdgcn_readfirstlane(r.mask);
        const unsigned int um = (fl >> mshift) & ((1u << WL::kUnitsPerWave) - 1u);
        if (um == 0u) continue;
        ThinX tx{};
        if constexpr (THIN) tx = uniform(sx[e]);
        float a[CP];
#pragma unroll
        for (int c = 0; c < CP; ++c) a[c] = r.amp[c];
        // The first unit of the mask assigns the partial sums (no zeroing);
        // the later ones add to them and are skipped when no lane of the
        // unit lies inside the truncation.
        float part[KP];
#pragma unroll
        for (int k = K; k < KP; ++k) part[k] = 0.f;
        bool any = false;
        auto unit = [&](auto uc, auto firstc) {
          constexpr int u = decltype(uc)::value, j = u / UX, i = u % UX;
          constexpr bool first = decltype(firstc)::value != 0;
          const float dy = (fy + (float)(UH * j)) - r.my;
          const float dx = (fx + (float)(UW * i)) - r.mx;
          float u1, u2;
          whiten<THIN>(r.l11, r.l12, r.l21, r.l22, tx, dx, dy, u1, u2);
          const float q = u1 * u1 + u2 * u2;
          const bool inside = q <= thr;
          const bool hit = __builtin_amdgcn_ballot_w64(inside) != 0ull;
          if (!first && !hit) return;
          any |= hit;
          const float w = inside ? __builtin_amdgcn_exp2f(-q) : 0.f;
          float h = G[j][i][0] * a[0];
#pragma unroll
          for (int c = 1; c < CP; ++c) h += G[j][i][c] * a[c];
          const float v = h * w;
          const float t1 = v * u1, t2 = v * u2;
          if constexpr (first) {
#pragma unroll
            for (int c = 0; c < CP; ++c) part[c] = G[j][i][c] * w;
            part[CP + 0] = t1;
            part[CP + 1] = t2;
            part[CP + 2] = t1 * u1;
            part[CP + 3] = t2 * u2;
            part[CP + 4] = t1 * u2;
          } else {
#pragma unroll
            for (int c = 0; c < CP; ++c) part[c] += G[j][i][c] * w;
            part[CP + 0] += t1;
            part[CP + 1] += t2;
            part[CP + 2] += t1 * u1;
            part[CP + 3] += t2 * u2;
            part[CP + 4] += t1 * u2;
          }
        };
        for_units_from_first<WL::kUnitsPerWave>(um, unit);
        if (!any) continue;
        // a thin entry with swapped rows accumulated S2, S1, S22, S11, S12
        const bool sw = THIN && (fl & kEntrySwap);
        auto swapped = [&](int sl) { return (sw && sl >= 0 && sl < 4) ? sl ^ 1 : sl; };
        if constexpr (kSplit) {
          // part[16..20] are the moments, part[21..23] zero
          const float tot = wave_reduce_transposed<16>(part, lane);
          const float tot_m = wave_reduce_transposed<8>(part + 16, lane);
          const int sm = swapped(slot_m);
          if (slot >= 0) unsafeAtomicAdd(sums + (unsigned)(r.row + slot), tot);
          if (sm >= 0) unsafeAtomicAdd(sums + (unsigned)(r.row + sm), tot_m);
        } else {
          float tot;
          if constexpr (kXpose) tot = wave_reduce_xpose<K, KP>(part, red, lane);
          else tot = wave_reduce_transposed<KP>(part, lane);
          const int sl = swapped(slot);
          if (sl >= 0) unsafeAtomicAdd(sums + (unsigned)(r.row + sl), tot);
        }
      }
    };
    run(IC<0>{}, 0, np);
    run(IC<1>{}, np, __builtin_amdgcn_readfirstlane(cnt));
  }
}

// grad_params holds the raw sums (S1, S2, S11, S22, S12, A_c) in its slots;
// apply the chain rule in place (fp64):
//   dmu = L^T (S1, S2) with L = [[c/s1, s/s1], [-s/s2, c/s2]],
//   ds1 = S11/s1, ds2 = S22/s2, dtheta = (s1/s2 - s2/s1) S12, da = A
// undoing the kappa scale of the whitened coordinates.  A Gaussian with an
// empty pixel box (culled, or with no pixel in the frame) is in no tile
// list: its row was zeroed and stays zero, so only its 8-byte box is read.
// When the raster met a non-finite dL/dI value (which it took as 0), the
// terms of such values on the Gaussian's support are added first: for
// every pixel of its box holding one inside the truncation (the
// definition's q, fp64), G_c w for the non-finite channels and, with
// X = sum of G_c a_c over them, X w times each moment.  The sums then carry
// the IEEE result of the full sum (finite + inf = inf, inf - inf = NaN).
__global__ __launch_bounds__(256) void k_finalize(const float *__restrict__ params,
                                                  const uint2 *__restrict__ boxes,
                                                  float *__restrict__ grad, long long BN, int N,
                                                  int C, const WsHeader *hdr,
                                                  const void *__restrict__ gimg, int ldo, int ooff,
                                                  int fmt, int H, int W, double k2) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= BN) return;
  const int P = 5 + C;
  float *o = grad + i * P;
  if (hdr->status & (kStatusOverflow | kStatusStale)) {   // no valid sums: NaN
    for (int c = 0; c < P; ++c) o[c] = __builtin_nanf("");
    return;
  }
  const uint2 bx = boxes[i];
  const int x0 = (int)(bx.x & 0xFFFFu), x1 = (int)(bx.x >> 16);
  const int y0 = (int)(bx.y & 0xFFFFu), y1 = (int)(bx.y >> 16);
  if (x0 > x1 || y0 > y1) return;
  const float *g = params + i * P;
  double sn, cs;
  sincos((double)g[4], &sn, &cs);
  const double s1 = g[2], s2 = g[3];
  double S1 = o[0], S2 = o[1], S11 = o[2], S22 = o[3], S12 = o[4];
  if (hdr->nonfinite) {
    const long long f = i / N;
    for (int y = y0; y <= y1; ++y) {
      for (int x = x0; x <= x1; ++x) {
        const size_t base = (((size_t)f * H + y) * W + x) * (size_t)ldo + ooff;
        bool any = false;
        for (int c = 0; c < C; ++c) any |= !__builtin_isfinite(load_image(gimg, base + c, fmt));
        if (!any) continue;
        const double dx = (x + 0.5) - (double)g[0], dy = (y + 0.5) - (double)g[1];
        const double z1 = (cs * dx + sn * dy) / s1, z2 = (-sn * dx + cs * dy) / s2;
        const double q = z1 * z1 + z2 * z2;
        if (!(q <= k2)) continue;
        const double w = exp(-0.5 * q);
        double X = 0.0;
        for (int c = 0; c < C; ++c) {
          const double gv = load_image(gimg, base + c, fmt);
          if (__builtin_isfinite(gv)) continue;
          o[5 + c] = (float)((double)o[5 + c] + gv * w);
          X += gv * (double)g[5 + c];
        }
        const double v = X * w, a1 = kKappa * z1, a2 = kKappa * z2;
        S1 += v * a1;
        S2 += v * a2;
        S11 += v * a1 * a1;
        S22 += v * a2 * a2;
        S12 += v * a1 * a2;
      }
    }
  }
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
    hdr->nonfinite = 0;
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

namespace {

struct RasterArgs {
  const GRec *recs;
  const ThinRec *thin;
  const float *params;
  const void *gimg;
  const int *tile_off;
  const int *list;
  int B, N, H, W, C, c0, cc;
  float thr;
  int nTx, nT;
  void *out;
  ImgView iv;
  const WsHeader *hdr;
  const int *order;
};

template <int CP, int UW, int UX, int UY, int FS>
void fwd_launch(const RasterArgs &a, hipStream_t st) {
  using WL = WaveLayout<UW, UX, UY>;
  dim3 grid((unsigned)xcd_grid(a.nT, a.B));
  PDR_TIMED(PDR_K_FORWARD_RASTER, st,
            hipLaunchKernelGGL((k_forward<CP, UW, UX, UY, FS>), grid, dim3(WL::kThreads * FS), 0,
                               st, a.recs, a.thin, a.params, a.tile_off, a.list, a.B, a.N, a.H,
                               a.W, a.C, a.c0, a.cc, a.thr, a.nTx, a.nT, a.out, a.iv, a.hdr,
                               a.order));
}

template <int CP, int UW, int UX, int UY>
void fwd_cp(const RasterArgs &a, hipStream_t st) {
  if constexpr (CP <= 4 && WaveLayout<UW, UX, UY>::kWaves == 1) {
    const int fs = forward_splits((long long)a.nT * a.B);
    if (fs >= 4) return fwd_launch<CP, UW, UX, UY, 4>(a, st);
    if (fs == 2) return fwd_launch<CP, UW, UX, UY, 2>(a, st);
  }
  fwd_launch<CP, UW, UX, UY, 1>(a, st);
}

template <int CP, int UW, int UX, int UY>
void bwd_cp(const RasterArgs &a, hipStream_t st) {
  using WL = WaveLayout<UW, UX, UY>;
  const int splits = backward_splits((long long)a.nT * a.B);
  dim3 grid((unsigned)(xcd_grid(a.nT, a.B) * splits));
  auto kern = splits > 1 ? k_backward<CP, UW, UX, UY, true> : k_backward<CP, UW, UX, UY, false>;
  PDR_TIMED(PDR_K_BACKWARD_RASTER, st,
            hipLaunchKernelGGL(kern, grid, dim3(WL::kThreads), 0, st,
                               a.recs, a.thin, a.params, a.gimg, a.tile_off, a.list, a.B, a.N,
                               a.H, a.W, a.C, a.c0, a.cc, a.thr, a.nTx, a.nT,
                               static_cast<float *>(a.out),
                               a.iv, const_cast<WsHeader *>(a.hdr), a.order, splits));
}

// Unit shape and units per wave (compile-time tuning knob): 8x8 quads,
// 2x2 per wave, one wave per tile (measured faster than 16x4 strips and
// than two or four waves per tile).  A wave always spans the tile's width.
#ifndef PDR_UNIT_W
#define PDR_UNIT_W 8
#define PDR_UNITS_X 2
#define PDR_UNITS_Y 2
#endif
template <bool BWD>
void dispatch(const RasterArgs &a, hipStream_t st) {
  constexpr int UW = PDR_UNIT_W, UX = PDR_UNITS_X, UY = PDR_UNITS_Y;
  const int cc = a.cc;
  if (cc <= 1) {
    BWD ? bwd_cp<1, UW, UX, UY>(a, st) : fwd_cp<1, UW, UX, UY>(a, st);
  } else if (cc == 2) {
    BWD ? bwd_cp<2, UW, UX, UY>(a, st) : fwd_cp<2, UW, UX, UY>(a, st);
  } else if (cc == 3) {
    BWD ? bwd_cp<3, UW, UX, UY>(a, st) : fwd_cp<3, UW, UX, UY>(a, st);
  } else if (cc == 4) {
    BWD ? bwd_cp<4, UW, UX, UY>(a, st) : fwd_cp<4, UW, UX, UY>(a, st);
  } else if (cc <= 8) {
    BWD ? bwd_cp<8, UW, UX, UY>(a, st) : fwd_cp<8, UW, UX, UY>(a, st);
  } else {
    BWD ? bwd_cp<16, UW, UX, UY>(a, st) : fwd_cp<16, UW, UX, UY>(a, st);
  }
}

float threshold(float radius) {
  // q' <= k^2 log2(e)/2, rounded once to fp32
  return (float)((double)radius * (double)radius * kKappa2);
}

RasterArgs raster_args(const float *params, int B, int N, int H, int W, int C, float radius,
                       void *ws, const Layout &L) {
  char *w = (char *)ws;
  RasterArgs a;
  a.recs = (const GRec *)(w + L.recs);
  a.thin = (const ThinRec *)(w + L.thin);
  a.params = params;
  a.gimg = nullptr;
  a.tile_off = (const int *)(w + L.tile_off);
  a.list = (const int *)(w + L.list);
  a.B = B; a.N = N; a.H = H; a.W = W; a.C = C;
  a.c0 = 0; a.cc = C;
  a.thr = threshold(radius);
  a.nTx = (W + kTileW - 1) / kTileW;
  a.nT = a.nTx * ((H + kTileH - 1) / kTileH);
  a.out = nullptr;
  a.iv = ImgView{C, 0, nullptr, nullptr, 0, PDR_FMT_F32};
  a.hdr = (const WsHeader *)(w + L.hdr);
  a.order = tile_order_on((long long)B * a.nT) ? (const int *)(w + L.order) : nullptr;
  return a;
}

}  // namespace

hipError_t launch_forward_raster(const float *params, void *image, int B, int N, int H, int W,
                                 int C, float radius, void *ws, const Layout &L, hipStream_t st,
                                 const float *pixel, int Cp, int fmt) {
  RasterArgs a = raster_args(params, B, N, H, W, C, radius, ws, L);
  a.out = image;
  a.iv = ImgView{Cp + C, Cp, nullptr, nullptr, Cp, fmt};
  for (int c0 = 0; c0 < C; c0 += 16) {
    a.c0 = c0;
    a.cc = C - c0 < 16 ? C - c0 : 16;
    a.iv.xin = (c0 == 0 && Cp > 0) ? pixel : nullptr;   // copied once
    dispatch<false>(a, st);
  }
  return hipGetLastError();
}

hipError_t launch_count_support(const float *params, int B, int N, int H, int W, int C,
                                float radius, void *ws, const Layout &L,
                                unsigned long long *count, hipStream_t st) {
  const RasterArgs a = raster_args(params, B, N, H, W, C, radius, ws, L);
  constexpr int UW = PDR_UNIT_W, UX = PDR_UNITS_X, UY = PDR_UNITS_Y;
  using WL = WaveLayout<UW, UX, UY>;
  hipLaunchKernelGGL(k_zero_count, dim3(1), dim3(1), 0, st, count);
  hipLaunchKernelGGL((k_count_support<UW, UX, UY>), dim3((unsigned)xcd_grid(a.nT, a.B)),
                     dim3(WL::kThreads), 0, st, a.recs, a.thin, a.params, a.tile_off, a.list, a.B,
                     a.N, a.H, a.W, a.C, a.thr, a.nTx, a.nT, count, a.hdr);
  return hipGetLastError();
}

hipError_t launch_backward(const float *params, const void *grad_image, float *grad_params, int B,
                           int N, int H, int W, int C, float radius, void *ws, const Layout &L,
                           bool check_stamp, hipStream_t st, float *grad_pixel, int Cp, int fmt) {
  RasterArgs a = raster_args(params, B, N, H, W, C, radius, ws, L);
  a.iv = ImgView{Cp + C, Cp, nullptr, nullptr, Cp, fmt};
  WsHeader *hdr = (WsHeader *)((char *)ws + L.hdr);
  long long BN = (long long)B * N, total = BN * (5 + C);
  long long zb = (total + 255) / 256;
  if (zb > 8192) zb = 8192;
  PDR_TIMED(PDR_K_ZERO, st,
            hipLaunchKernelGGL(k_zero_verify, dim3((unsigned)zb), dim3(256), 0, st, grad_params,
                               total, hdr, check_stamp ? 1 : 0, B, N, H, W, C, radius,
                               (unsigned long long)(uintptr_t)params));
  a.gimg = grad_image;
  a.out = grad_params;
  for (int c0 = 0; c0 < C; c0 += 16) {
    a.c0 = c0;
    a.cc = C - c0 < 16 ? C - c0 : 16;
    a.iv.xout = (c0 == 0 && Cp > 0) ? grad_pixel : nullptr;   // copied once
    dispatch<true>(a, st);
  }
  PDR_TIMED(PDR_K_FINALIZE, st,
            hipLaunchKernelGGL(k_finalize, dim3((unsigned)((BN + 255) / 256)), dim3(256), 0, st,
                               params, (const uint2 *)((char *)ws + L.boxes), grad_params, BN, N,
                               C, (const WsHeader *)hdr, grad_image, Cp + C, Cp, fmt, H, W,
                               (double)radius * (double)radius));
  return hipGetLastError();
}

}  // namespace pdr
