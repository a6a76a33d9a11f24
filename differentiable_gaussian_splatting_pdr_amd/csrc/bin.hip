// bin.hip -- per-Gaussian preprocessing and tile binning.
//
//  k_preprocess   one thread per Gaussian: validity, fp64 pixel bounding box
//                 of the truncated ellipse q <= k^2, whitening rows (and the
//                 compensation constants of thin Gaussians).
//  k_bin<false,M,X> per (frame, tile group): per-tile overlap counts.
//  k_count_scan     the groups' first list offsets (a linear scan of the
//                   group totals) and the tile order's cursors.
//  k_bin<true,M,X>  per (frame, tile group): the per-tile lists, ascending
//                   Gaussian index, at the scanned offsets.
//
// A tile group holds a band of tile rows (or, when a batch has too few tile
// rows to fill the GPU, a column chunk of a one-row band) and walks the
// frame's Gaussians in chunks (consecutive Gaussians, or, M = true, the
// group's members); for each
// chunk it builds an LDS bit matrix [tile][Gaussian] of box overlaps and
// compacts every tile's bit row with a wave scan.  The lists are thus
// produced in ascending order with no sort and no global atomics.
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

// One workgroup per 256 Gaussians: their parameter rows (5 + C floats each)
// are read with coalesced loads, the first five values of every row staged
// in LDS and any non-finite value flagged, then each thread builds one
// Gaussian's record.
constexpr int kZeroBlocks = 32;   // preprocess blocks at least (for clearing the order histogram)

__global__ __launch_bounds__(256) void k_preprocess(const float *__restrict__ params, int BN, int C,
                                                    FastDiv pdiv, int H, int W, float radius,
                                                    GRec *__restrict__ recs,
                                                    ThinRec *__restrict__ thin,
                                                    uint2 *__restrict__ boxes, WsHeader *hdr,
                                                    int stamp_N, unsigned long long stamp_ptr,
                                                    int *__restrict__ ohist) {
  __shared__ float s5[5][256];
  __shared__ int bad[256];
  const int tid = threadIdx.x;
  const int g0 = blockIdx.x * 256;
  const int i = g0 + tid;
  // the tile-order histogram the binning's count pass fills, if any (the
  // grid then has at least kZeroBlocks blocks; those past the Gaussians only
  // clear it)
  if (ohist)
    for (int j = i; j < 8 * kOrderBuckets; j += gridDim.x * 256) ohist[j] = 0;
  if (g0 >= BN) return;  // uniform per block
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
  bad[tid] = 0;
  __syncthreads();
  const int ng = min(256, BN - g0);
  const uint32_t P = pdiv.d;
  const uint32_t tot = (uint32_t)ng * P;
  const float *src = params + (size_t)g0 * P;
  for (uint32_t e = tid; e < tot; e += 256) {
    const float v = src[e];
    const uint32_t g = fdiv(e, pdiv);
    const uint32_t k = e - g * P;
    if (k < 5) s5[k][g] = v;
    if (!isfinite(v)) bad[g] = 1;
  }
  __syncthreads();
  if (tid >= ng) return;
  float mx = s5[0][tid], my = s5[1][tid], s1 = s5[2][tid], s2 = s5[3][tid], th = s5[4][tid];
  const bool ok = !bad[tid] && s1 > 0.f && s2 > 0.f;
  GRec r;
  r.mx = mx;
  r.my = my;
  r.l11 = r.l12 = r.l21 = r.l22 = 0.f;
  r.bx = kEmptyBox;
  r.by = kEmptyBox;
  if (ok) {
    double L[4], sn, cs;
    whitening_rows(th, s1, s2, L, &sn, &cs);
    int b[4];
    pixel_box(mx, my, s1, s2, cs, sn, (double)radius, H, W, b);
    if (b[0] <= b[1] && b[2] <= b[3]) {
      r.bx = (unsigned)b[0] | ((unsigned)b[1] << 16);
      r.by = (unsigned)b[2] | ((unsigned)b[3] << 16);
    }
    r.l11 = clamp_to_float(L[0]);
    r.l12 = clamp_to_float(L[1]);
    r.l21 = clamp_to_float(L[2]);
    r.l22 = clamp_to_float(L[3]);
    if (is_thin(r.l11, r.l12, r.l21, r.l22)) {
      const float l32[4] = {r.l11, r.l12, r.l21, r.l22};
      thin[i] = make_thin_rec(mx, my, L, l32);
    }
  }
  recs[i] = r;
  boxes[i] = make_uint2(r.bx, r.by);
}

// Sum of a long long over the workgroup (all threads receive it).
__device__ __forceinline__ long long block_sum_ll(long long v, long long *red) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  long long t = 0;
  for (int w = 0; w < kBinThreads / kWave; ++w) t += red[w];
  __syncthreads();
  return t;
}

// Between the count and write passes, one launch of 9 workgroups:
//  * workgroups 0-7 (when the rasters take the tile order): XCD range r's
//    order-key histogram becomes cursors -- its exclusive scan (keys
//    ascending: longest first) plus the range's first slot, so that each
//    entry is the next free position of its key in order[];
//  * workgroup 8: the group totals gtot[0 .. ngroups) become their exclusive
//    prefix, each write group's first list offset (clamped to int: any
//    offset past that overflows the list capacity), in one linear pass; the
//    pair total goes to the header with the overflow flag (a fresh binning
//    clears any earlier overflow or stale flag).
constexpr int kScanPer = 8;   // group totals per thread per round
constexpr int kOrderPer = kOrderBuckets / kBinThreads;
static_assert(kOrderBuckets % kBinThreads == 0, "whole keys per thread");
__global__ __launch_bounds__(kBinThreads) void k_count_scan(int *__restrict__ gtot,
                                                            long long ngroups, long long cap,
                                                            WsHeader *hdr,
                                                            int *__restrict__ ohist,
                                                            unsigned int total_tiles) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (blockIdx.x < 8) {
    if (!ohist) return;
    __shared__ int wtot[kBinThreads / kWave];
    const int r = blockIdx.x;
    const unsigned int per = (total_tiles + 7u) >> 3;
    int *h = ohist + r * kOrderBuckets;
    int v[kOrderPer], t = 0;
#pragma unroll
    for (int k = 0; k < kOrderPer; ++k) {
      v[k] = h[tid * kOrderPer + k];
      t += v[k];
    }
    const int incl = wave_incl_scan(t);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int wex = 0;
    for (int w = 0; w < wave; ++w) wex += wtot[w];
    int e = (int)((unsigned int)r * per) + wex + incl - t;
#pragma unroll
    for (int k = 0; k < kOrderPer; ++k) {
      h[tid * kOrderPer + k] = e;
      e += v[k];
    }
    return;
  }
  __shared__ long long wtl[kBinThreads / kWave];
  long long carry = 0;
  for (long long r0 = 0; r0 < ngroups; r0 += (long long)kBinThreads * kScanPer) {
    const long long i0 = r0 + (long long)tid * kScanPer;
    int v[kScanPer];
    long long t = 0;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      v[k] = i0 + k < ngroups ? gtot[i0 + k] : 0;
      t += v[k];
    }
    long long incl = t;   // inclusive scan over the wave (64-bit)
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const long long o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane == 63) wtl[wave] = incl;
    __syncthreads();
    long long wex = 0, rtot = 0;
    for (int w = 0; w < kBinThreads / kWave; ++w) {
      wex += w < wave ? wtl[w] : 0;
      rtot += wtl[w];
    }
    long long e = carry + wex + incl - t;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      if (i0 + k < ngroups) gtot[i0 + k] = (int)min(e, 0x7fffffffLL);
      e += v[k];
    }
    carry += rtot;
    __syncthreads();  // wtl is rewritten by the next round
  }
  if (tid == 0) {
    hdr->total = carry;
    hdr->cap = cap;
    hdr->status = (carry > cap || carry > 0x7fffffffLL) ? kStatusOverflow : 0;
  }
}

// LDS bit matrix binning.  Grid: G groups x B frames (1D, XCD-aware); a group
// is a band of gh whole tile rows, or with ncc > 1 column chunks one tile row
// of cw tiles (the last chunk narrower).  Either way its tiles are one
// contiguous run of the frame's row-major tile order.  Dynamic LDS:
// Tg * (NC / 32) words of bits (NC a multiple of 64), then, with MEMBERS, NC
// member indices.
//
// A chunk is a set of at most NC Gaussians in ascending index order; each
// sets, in its column, the bits of the band's tiles its box overlaps, each
// tile's bit row is compacted with a wave scan and the columns map back to
// Gaussian indices.  Lists thus come out ascending with no sort and no
// global atomics.  Two ways of forming chunks:
//  MEMBERS = false  chunk = NC consecutive Gaussians of the frame, loaded one
//                   chunk ahead; every tile row compacts all NC columns.
//  MEMBERS = true   the group scans the frame's boxes in segments (loaded one
//                   segment ahead) and gathers the group's members -- the
//                   Gaussians whose box meets its tiles -- into an LDS list in
//                   index order (wave ballots, a prefix over waves); NC
//                   members form a chunk.  A band then pays for bit setting
//                   and compaction on its own members only, which wins when
//                   a frame has many bands.
//
// Count pass (WRITE = false): per-tile counts -- one LDS atomic add per
// (box, group tile) overlap, over the boxes the group would scan -- and the
// group's total.
// Write pass (WRITE = true): the group's base offset is the exclusive
// prefix of the group totals (frame-major, bands top to bottom) that
// k_count_scan left in gtot; an exclusive scan (wave64 DPP scan) of its
// tiles' counts gives their offsets; then the lists are written through the
// chunks above.  A tile's list length is the number of boxes that meet it
// either way.
constexpr int kSegSlots = 4;   // boxes per thread per member-scan segment

template <bool WRITE, bool MEMBERS, bool COLS, bool ROWL = false>
__global__ __launch_bounds__(kBinThreads) void k_bin(const uint2 *__restrict__ boxes, int B, int N,
                                                     int nTx, int nTy, int gh, int ncc, int cw,
                                                     int G, int NC, int *__restrict__ counts,
                                                     int *__restrict__ gtot,
                                                     int *__restrict__ tile_off,
                                                     int *__restrict__ list, long long cap,
                                                     WsHeader *hdr, int *__restrict__ ohist,
                                                     int *__restrict__ order,
                                                     const int *__restrict__ rlist = nullptr,
                                                     const int *__restrict__ fstart = nullptr,
                                                     long long rcap = 0) {
  static_assert(!ROWL || MEMBERS, "row lists feed the member scan");
  extern __shared__ unsigned int dyn[];
  __shared__ int base[kMaxGroupTiles];
  __shared__ long long red[kBinThreads / kWave];
  __shared__ int wtot[kBinThreads / kWave];
  __shared__ int wcnt[kSegSlots][kBinThreads / kWave];
  int b, g;  // frame, group: all groups of a frame on one XCD, so its boxes stay in that L2
  if (!xcd_frame_item(blockIdx.x, G, B, &b, &g)) return;
  // group g = (band, column chunk): tile rows [ty0, ty0 + ah), tile columns
  // [cx0, cx0 + aw); with more than one chunk a band is one tile row, so a
  // group's tiles are always one contiguous run of the frame's tile order
  const int band = COLS ? g / ncc : g, chunk = COLS ? g - band * ncc : 0;
  const int ty0 = band * gh;
  const int ah = min(gh, nTy - ty0);
  const int cx0 = COLS ? chunk * cw : 0;
  const int aw = COLS ? min(cw, nTx - cx0) : nTx;
  const int Tg = aw * ah;
  const int nT = nTx * nTy;
  const size_t t0 = (size_t)b * nT + (size_t)ty0 * nTx + cx0;  // first tile of the group
  const int words = NC >> 5;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned int *bits = dyn;
  int *mem = (int *)(dyn + (size_t)Tg * words);  // MEMBERS only

  // ROWL: the member scan walks the group's tile row's list (gh = 1).  If
  // the row lists did not fit the workspace (they were not written), it
  // scans all of the frame's boxes instead: slower, same lists and counts.
  const int *rl = nullptr;
  int rn = N;
  if constexpr (ROWL) {
    long long part = 0, all = 0;
    for (int f = tid; f < B; f += kBinThreads) {
      const long long t = fstart[(size_t)f * (nTy + 1) + nTy];
      part += f < b ? t : 0;
      all += t;
    }
    const long long fbase = block_sum_ll(part, red);
    const long long rows_all = block_sum_ll(all, red);
    // (a frame's row count saturates at 2^31 - 1)
    if (rows_all <= rcap && rows_all < 0x7fffffffLL) {
      const int *fs = fstart + (size_t)b * (nTy + 1);
      rl = rlist + fbase + fs[ty0];
      rn = fs[ty0 + 1] - fs[ty0];
    }
  }

  if (WRITE) {
    // base of this group: the exclusive prefix of the group totals, which
    // the count pass's last group left in gtot
    const long long gbase = gtot[(size_t)b * G + g];
    // exclusive scan of the group's tile counts (2 * kBinThreads >= Tg)
    const int c0 = 2 * tid < Tg ? counts[t0 + 2 * tid] : 0;
    const int c1 = 2 * tid + 1 < Tg ? counts[t0 + 2 * tid + 1] : 0;
    const int incl = wave_incl_scan(c0 + c1);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int wex = 0, gsum = 0;
    for (int w = 0; w < kBinThreads / kWave; ++w) {
      wex += w < wave ? wtot[w] : 0;
      gsum += wtot[w];
    }
    const long long e0 = gbase + wex + incl - (c0 + c1);
    if (2 * tid < Tg) {
      tile_off[t0 + 2 * tid] = (int)min(e0, 0x7fffffffLL);
      base[2 * tid] = (int)min(e0, 0x7fffffffLL);
    }
    if (2 * tid + 1 < Tg) {
      tile_off[t0 + 2 * tid + 1] = (int)min(e0 + c0, 0x7fffffffLL);
      base[2 * tid + 1] = (int)min(e0 + c0, 0x7fffffffLL);
    }
    // longest-first raster order: each tile takes the next slot of its
    // (XCD range, length bucket); the cursors come from k_count_scan
    if (ohist) {
      const unsigned int total = (unsigned int)B * (unsigned int)nT;
      for (int k = 0; k < 2; ++k) {
        if (2 * tid + k >= Tg) break;
        const unsigned int gt = (unsigned int)(t0 + 2 * tid + k);
        order[atomicAdd(&ohist[order_slot(gt, total, k ? c1 : c0)], 1)] = (int)gt;
      }
    }
    const long long gend = gbase + gsum;
    const bool limit = gend > cap || gend > 0x7fffffffLL;
    if (tid == 0 && b == B - 1 && g == G - 1)
      tile_off[(size_t)B * nT] = (int)min(hdr->total, 0x7fffffffLL);
    if (limit) return;  // uniform: this group's lists do not fit
  } else {
    for (int lt = tid; lt < Tg; lt += kBinThreads) base[lt] = 0;
  }

  const uint2 *fb = boxes + (size_t)b * N;

  // Column j of the chunk holds box bx: set its bits in the band's tiles.
  auto set_bits = [&](int j, uint2 bx) {
    const int x0 = (int)(bx.x & 0xffffu), x1 = (int)(bx.x >> 16);
    const int y0 = (int)(bx.y & 0xffffu), y1 = (int)(bx.y >> 16);
    if (x0 > x1) return;
    const int ux0 = COLS ? max(x0 >> kTileShiftX, cx0) : x0 >> kTileShiftX;
    const int ux1 = COLS ? min(x1 >> kTileShiftX, cx0 + aw - 1) : x1 >> kTileShiftX;
    const int uy0 = max(y0 >> kTileShiftY, ty0), uy1 = min(y1 >> kTileShiftY, ty0 + ah - 1);
    const unsigned int bit = 1u << (j & 31);
    const int wi = j >> 5;
    for (int ty = uy0; ty <= uy1; ++ty)
      for (int tx = ux0; tx <= ux1; ++tx)
        atomicOr(&bits[((ty - ty0) * aw + (tx - cx0)) * words + wi], bit);
  };
  // Compaction of the first `used` bit words of every tile row (a wave owns
  // every eighth tile from its own index on), which it leaves cleared;
  // column j maps to Gaussian col(j).
  auto compact = [&](int used, auto col) {
    for (int lt = wave; lt < Tg; lt += kBinThreads / kWave) {
      int run = base[lt];
      unsigned int *row = bits + (size_t)lt * words;
      for (int seg = 0; seg < used; seg += 2 * kWave) {
        const int w0 = seg + 2 * lane;  // words even: w0 + 1 < words
        unsigned long long m = 0ull;
        if (w0 < used) {
          m = (unsigned long long)row[w0] | ((unsigned long long)row[w0 + 1] << 32);
          row[w0] = 0u;
          row[w0 + 1] = 0u;
        }
        const int c = __popcll(m);
        const int incl = wave_incl_scan(c);
        if (WRITE) {
          int pos = run + incl - c;
          const int nb = w0 * 32;
          while (m) {
            const int k = __ffsll((long long)m) - 1;
            list[pos++] = col(nb + k);
            m &= m - 1ull;
          }
        }
        run += wave_read(incl, 63);
      }
      if (lane == 0) base[lt] = run;
    }
  };

  if constexpr (!WRITE) {
    // The count pass needs no order: every (box, group tile) overlap adds
    // one to the tile's count -- the same integers the write pass's bit
    // matrix yields, with no matrix and no compaction.
    __syncthreads();  // base cleared
    for (int j0 = 0; j0 < rn; j0 += kSegSlots * kBinThreads) {
      // kSegSlots boxes per thread in flight at once (list entries first)
      int n[kSegSlots];
      uint2 bx[kSegSlots];
#pragma unroll
      for (int k = 0; k < kSegSlots; ++k) {
        const int j = j0 + k * kBinThreads + tid;
        n[k] = j;
        if constexpr (ROWL) n[k] = (rl && j < rn) ? rl[j] : j;
      }
#pragma unroll
      for (int k = 0; k < kSegSlots; ++k)
        bx[k] = j0 + k * kBinThreads + tid < rn ? fb[n[k]] : make_uint2(kEmptyBox, kEmptyBox);
#pragma unroll
      for (int k = 0; k < kSegSlots; ++k) {
        const int x0 = (int)(bx[k].x & 0xffffu), x1 = (int)(bx[k].x >> 16);
        const int y0 = (int)(bx[k].y & 0xffffu), y1 = (int)(bx[k].y >> 16);
        if (x0 > x1) continue;
        const int ux0 = max(x0 >> kTileShiftX, cx0), ux1 = min(x1 >> kTileShiftX, cx0 + aw - 1);
        const int uy0 = max(y0 >> kTileShiftY, ty0), uy1 = min(y1 >> kTileShiftY, ty0 + ah - 1);
        for (int ty = uy0; ty <= uy1; ++ty)
          for (int tx = ux0; tx <= ux1; ++tx) atomicAdd(&base[(ty - ty0) * aw + (tx - cx0)], 1);
      }
    }
  } else {
    for (int w = tid; w < Tg * words; w += kBinThreads) bits[w] = 0u;

    if constexpr (!MEMBERS) {
      // chunks of NC consecutive Gaussians, loaded all at once one chunk ahead
      constexpr int kPer = kMaxChunk / kBinThreads;
      uint2 nxt[kPer];
      auto load_chunk = [&](int c) {
  #pragma unroll
        for (int k = 0; k < kPer; ++k) {
          const int i = tid + k * kBinThreads;
          nxt[k] = (i < NC && c + i < N) ? fb[c + i] : make_uint2(kEmptyBox, kEmptyBox);
        }
      };
      load_chunk(0);
      for (int c0 = 0; c0 < N; c0 += NC) {
        uint2 cur[kPer];
  #pragma unroll
        for (int k = 0; k < kPer; ++k) cur[k] = nxt[k];
        __syncthreads();  // bits clear
        if (c0 + NC < N) load_chunk(c0 + NC);
  #pragma unroll
        for (int k = 0; k < kPer; ++k) set_bits(tid + k * kBinThreads, cur[k]);
        __syncthreads();
        compact(min(NC, N - c0 + 31) >> 5, [&](int j) { return c0 + j; });
      }
    } else {
      // the members [0, cnt) form a chunk
      auto flush = [&](int cnt) {
        __syncthreads();  // member list complete, bits clear
        for (int j = tid; j < cnt; j += kBinThreads) set_bits(j, fb[mem[j]]);
        __syncthreads();
        compact((cnt + 31) >> 5, [&](int j) { return mem[j]; });
        __syncthreads();  // the member list is refilled next
      };
      bool direct = false;
      if constexpr (ROWL && !COLS) direct = rl != nullptr;
      if (direct) {
        // a whole tile row: every entry of the row's list meets the group
        for (int c0 = 0; c0 < rn; c0 += NC) {
          const int cnt = min(NC, rn - c0);
          for (int j = tid; j < cnt; j += kBinThreads) mem[j] = rl[c0 + j];
          flush(cnt);
        }
      } else {
        const int S = min(NC, kSegSlots * kBinThreads);  // boxes per segment
        uint2 nxt[kSegSlots];
        int nid[kSegSlots];   // ROWL: the Gaussian indices of the prefetched boxes
        auto load_seg = [&](int s0) {
    #pragma unroll
          for (int k = 0; k < kSegSlots; ++k) {
            const int o = k * kBinThreads + tid;
            const bool v = o < S && s0 + o < rn;
            if constexpr (ROWL) {
              nid[k] = v ? (rl ? rl[s0 + o] : s0 + o) : 0;
              nxt[k] = v ? fb[nid[k]] : make_uint2(kEmptyBox, kEmptyBox);
            } else {
              nxt[k] = v ? fb[s0 + o] : make_uint2(kEmptyBox, kEmptyBox);
            }
          }
        };
        load_seg(0);
        int cnt = 0;  // members gathered for the current chunk (uniform)
        for (int s0 = 0; s0 < rn; s0 += S) {
          bool in[kSegSlots];
          unsigned long long bal[kSegSlots];
          int cid[kSegSlots];
    #pragma unroll
          for (int k = 0; k < kSegSlots; ++k) {
            cid[k] = ROWL ? nid[k] : s0 + k * kBinThreads + tid;
            const uint2 bx = nxt[k];
            const int x0 = (int)(bx.x & 0xffffu), x1 = (int)(bx.x >> 16);
            const int y0 = (int)(bx.y & 0xffffu), y1 = (int)(bx.y >> 16);
            in[k] = x0 <= x1 && (y0 >> kTileShiftY) < ty0 + ah && (y1 >> kTileShiftY) >= ty0 &&
                    (!COLS || ((x0 >> kTileShiftX) < cx0 + aw && (x1 >> kTileShiftX) >= cx0));
            bal[k] = __builtin_amdgcn_ballot_w64(in[k]);
            if (lane == 0) wcnt[k][wave] = __popcll(bal[k]);
          }
          if (s0 + S < rn) load_seg(s0 + S);
          __syncthreads();
          // members of this segment, in index order (slot-major, then wave, lane)
          int total = 0, before[kSegSlots];
    #pragma unroll
          for (int k = 0; k < kSegSlots; ++k) {
            int wsum = 0, wpre = 0;
            for (int w = 0; w < kBinThreads / kWave; ++w) {
              wpre += w < wave ? wcnt[k][w] : 0;
              wsum += wcnt[k][w];
            }
            before[k] = total + wpre;
            total += wsum;
          }
          if (cnt + total > NC) {  // total <= S <= NC
            flush(cnt);
            cnt = 0;
          }
          const unsigned long long lt_mask = (1ull << lane) - 1ull;
    #pragma unroll
          for (int k = 0; k < kSegSlots; ++k)
            if (in[k]) mem[cnt + before[k] + __popcll(bal[k] & lt_mask)] = cid[k];
          cnt += total;
          __syncthreads();  // wcnt is rewritten by the next segment
        }
        if (cnt > 0) flush(cnt);
      }
    }
  }
  __syncthreads();
  if (!WRITE) {
    long long part = 0;
    const unsigned int total = (unsigned int)B * (unsigned int)nT;
    for (int lt = tid; lt < Tg; lt += kBinThreads) {
      counts[t0 + lt] = base[lt];
      part += base[lt];
      // histogram of the tiles' order keys per XCD range
      if (ohist) atomicAdd(&ohist[order_slot((unsigned int)(t0 + lt), total, base[lt])], 1);
    }
    const long long tot = block_sum_ll(part, red);
    if (tid == 0) gtot[(size_t)b * G + g] = (int)min(tot, 0x7fffffffLL);
  }
}

// ----------------------------------------------------------------------------
// Per-row member lists (first level of the two-level binning).
//
// k_rows<false>: per (frame, block of RB Gaussians): an LDS bit matrix
//   [tile row][Gaussian of the block] of box overlaps; the popcount of each
//   row is stored at rcnt[(frame * nTy + row) * nblk + block].
// k_rowscan, k_rowstart: rcnt becomes each block's offset within its row's
//   list, fstart[frame][row] the frame-local start of each row's list and
//   fstart[frame][nTy] the frame's total.
// k_rows<true>: the same bit matrix; each row's members are compacted into
//   rlist at (frames before) + (row start) + rcnt, so every row's list
//   holds ascending Gaussian indices (blocks in order, bits in order).
//   Nothing is written if the row pairs of all frames exceed the row list
//   capacity rcap.
template <bool WRITE>
__global__ __launch_bounds__(kBinThreads) void k_rows(const uint2 *__restrict__ boxes, int B,
                                                      int N, int nTy, int RB, int nblk,
                                                      int *__restrict__ rcnt,
                                                      const int *__restrict__ fstart,
                                                      int *__restrict__ rlist, long long rcap) {
  extern __shared__ unsigned int rbits[];
  __shared__ long long red[kBinThreads / kWave];
  int b, k;
  if (!xcd_frame_item(blockIdx.x, nblk, B, &b, &k)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int words = RB >> 5;
  const int j0 = k * RB;
  const int nj = min(RB, N - j0);
  long long fbase = 0;
  if (WRITE) {
    long long part = 0, all = 0;
    for (int f = tid; f < B; f += kBinThreads) {
      const long long t = fstart[(size_t)f * (nTy + 1) + nTy];
      part += f < b ? t : 0;
      all += t;
    }
    fbase = block_sum_ll(part, red);
    const long long rows_all = block_sum_ll(all, red);
    if (rows_all > rcap || rows_all >= 0x7fffffffLL) return;  // uniform: the row lists do not fit
  }
  for (int w = tid; w < nTy * words; w += kBinThreads) rbits[w] = 0u;
  __syncthreads();
  const uint2 *fb = boxes + (size_t)b * N + j0;
  for (int jj = tid; jj < nj; jj += kBinThreads) {
    const uint2 bx = fb[jj];
    const int x0 = (int)(bx.x & 0xffffu), x1 = (int)(bx.x >> 16);
    const int y0 = (int)(bx.y & 0xffffu), y1 = (int)(bx.y >> 16);
    if (x0 > x1 || y0 > y1) continue;
    const unsigned int bit = 1u << (jj & 31);
    for (int r = y0 >> kTileShiftY; r <= (y1 >> kTileShiftY); ++r)
      atomicOr(&rbits[r * words + (jj >> 5)], bit);
  }
  __syncthreads();
  // a wave per row: rows wave, wave + 8, ...
  for (int r = wave; r < nTy; r += kBinThreads / kWave) {
    const size_t ci = ((size_t)b * nTy + r) * nblk + k;
    const unsigned int *row = rbits + (size_t)r * words;
    int run = WRITE ? (int)(fbase + fstart[(size_t)b * (nTy + 1) + r] + rcnt[ci]) : 0;
    for (int seg = 0; seg < words; seg += 2 * kWave) {
      const int w0 = seg + 2 * lane;  // words even
      const unsigned long long m =
          w0 < words ? ((unsigned long long)row[w0] | ((unsigned long long)row[w0 + 1] << 32)) : 0ull;
      const int c = __popcll(m);
      const int incl = wave_incl_scan(c);
      if (WRITE) {
        int pos = run + incl - c;
        unsigned long long mm = m;
        while (mm) {
          const int q = __ffsll((long long)mm) - 1;
          rlist[pos++] = j0 + w0 * 32 + q;
          mm &= mm - 1ull;
        }
      }
      run += wave_read(incl, 63);
    }
    if (!WRITE && lane == 0) rcnt[ci] = run;
  }
}

// One wave per (frame, tile row): exclusive scan of the row's nblk block
// counts in place (each lane takes kRowScanPer consecutive counts per
// round), the row's total into fstart[frame][row].
constexpr int kRowScanPer = 8;
__global__ __launch_bounds__(kWave) void k_rowscan(int *__restrict__ rcnt, int B, int nTy, int nblk,
                                                   int *__restrict__ fstart) {
  int b, r;
  if (!xcd_frame_item(blockIdx.x, nTy, B, &b, &r)) return;
  const int lane = threadIdx.x;
  int *c = rcnt + ((size_t)b * nTy + r) * nblk;
  int run = 0;
  for (int c0 = 0; c0 < nblk; c0 += kWave * kRowScanPer) {
    const int i0 = c0 + lane * kRowScanPer;
    int v[kRowScanPer], t = 0;
#pragma unroll
    for (int k = 0; k < kRowScanPer; ++k) {
      v[k] = i0 + k < nblk ? c[i0 + k] : 0;
      t += v[k];
    }
    const int incl = wave_incl_scan(t);
    int e = run + incl - t;
#pragma unroll
    for (int k = 0; k < kRowScanPer; ++k) {
      if (i0 + k < nblk) c[i0 + k] = e;
      e += v[k];
    }
    run += wave_read(incl, 63);
  }
  if (lane == 0) fstart[(size_t)b * (nTy + 1) + r] = run;
}

// One workgroup per frame: the row totals in fstart[frame][0..nTy) become
// the rows' list starts (exclusive scan, kRowStartPer rows per thread and
// round), fstart[frame][nTy] the frame's total, saturated at 2^31 - 1.
constexpr int kRowStartPer = 4;
__global__ __launch_bounds__(kBinThreads) void k_rowstart(int nTy, int *__restrict__ fstart) {
  __shared__ long long wtot[kBinThreads / kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int *fs = fstart + (size_t)blockIdx.x * (nTy + 1);
  long long carry = 0;
  for (int r0 = 0; r0 < nTy; r0 += kBinThreads * kRowStartPer) {
    const int i0 = r0 + tid * kRowStartPer;
    long long v[kRowStartPer], t = 0;
#pragma unroll
    for (int k = 0; k < kRowStartPer; ++k) {
      v[k] = i0 + k < nTy ? fs[i0 + k] : 0;
      t += v[k];
    }
    long long incl = t;  // wave inclusive scan (64-bit, shuffles)
    for (int d = 1; d < kWave; d <<= 1) {
      const long long o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    long long wex = 0, tot = 0;
    for (int w = 0; w < kBinThreads / kWave; ++w) {
      wex += w < wave ? wtot[w] : 0;
      tot += wtot[w];
    }
    long long e = carry + wex + incl - t;
#pragma unroll
    for (int k = 0; k < kRowStartPer; ++k) {
      if (i0 + k < nTy) fs[i0 + k] = (int)min(e, 0x7fffffffLL);
      e += v[k];
    }
    carry += tot;
    __syncthreads();  // wtot is rewritten by the next round
  }
  if (tid == 0) fs[nTy] = (int)min(carry, 0x7fffffffLL);
}

// ----------------------------------------------------------------------------
// host launchers

// Tile groups: bands of whole tile rows whose bit rows (Tg x NC bits) -- and,
// with a member list, its NC indices -- fit the LDS budget; within that,
// frames are split into more bands so that the grid has about
// kBinTargetGroups workgroups (every group scans the frame's boxes, which
// stay in L2).  When a whole batch has fewer than kBinChunkBelow tile rows
// (a few very wide frames), bands are one tile row and are also cut into
// column chunks of at least kBinMinChunkTiles tiles, aiming at
// kBinChunkTarget groups: every group still scans all of its frame's boxes,
// so chunks only pay where a full tile row would force a narrow bit matrix
// (NC limited by the LDS) and long compactions -- measured on MI355X 290 ->
// 45 us of binning for one 20 x 16384 frame, but 0.77 -> 7.2 ms for one
// 2048 x 2048 frame with 262144 Gaussians had the rule chunked it.
// Integer arithmetic throughout: NC must be a multiple of 64.
struct BinGroups {
  int gh;   // tile rows per band
  int ncc;  // column chunks per band
  int cw;   // tiles per chunk (the last may be narrower)
  int NC;   // bit-matrix columns (Gaussians per chunk of the scan)
  int G;    // groups per frame
};

static BinGroups choose_groups(int B, int N, int nTx, int nTy, bool members) {
  BinGroups r;
  const long long rows_all = (long long)B * nTy;
  int c = 1;
  if (rows_all < kBinChunkBelow && nTx >= 2 * kBinMinChunkTiles) {
    c = (int)((kBinChunkTarget + rows_all - 1) / rows_all);
    if (c > nTx / kBinMinChunkTiles) c = nTx / kBinMinChunkTiles;
  }
  r.cw = (nTx + c - 1) / c;
  r.ncc = (nTx + r.cw - 1) / r.cw;
  long long nc = ((long long)N + 63) / 64 * 64;
  if (nc > kMaxChunk) nc = kMaxChunk;
  // one column of a full group row costs cw bits, plus 32 for its member index
  const long long row_max = kBinLdsBytes * 8 / (r.cw + (members ? 32 : 0)) / 64 * 64;
  if (nc > row_max) nc = row_max;
  r.NC = (int)nc;
  long long rows = (kBinLdsBytes - (members ? nc * 4 : 0)) * 8 / (nc * r.cw);
  if (rows > kMaxGroupTiles / r.cw) rows = kMaxGroupTiles / r.cw;
  if (rows > nTy) rows = nTy;
  if (r.ncc > 1) {
    rows = 1;   // chunked bands are single tile rows (contiguous tile runs)
  } else {
    int want = (int)((kBinTargetGroups + B - 1) / B);  // bands per frame for a full grid
    if (want > 1) {
      int rr = (nTy + want - 1) / want;
      if (rr < rows) rows = rr;
    }
  }
  r.gh = rows < 1 ? 1 : (int)rows;
  r.G = (nTy + r.gh - 1) / r.gh * r.ncc;
  return r;
}

// Member lists pay when a frame has many groups (a group meets a small
// share of its boxes) and the consecutive chunks' compaction is long:
// every group compacts N * Tg / 32 bit words, which the member lists cut
// to the group's share.  Measured on MI355X: 26% faster binning at 16
// bands and N * Tg = 2^22, a tie at 32 bands and 2^18, slower below.
static bool member_rule(int N, const BinGroups &bg) {
  return bg.G >= kBinMemberBands && (long long)N * bg.cw * bg.gh >= kBinMemberWords * 32;
}

// Second level of the two-level binning: one tile row per group, cut into
// column chunks so that the grid has about kBinRowTargetGroups workgroups (a
// chunk scans only its row's list, so chunks cost no rescans of the frame).
static BinGroups row_groups(int B, int N, int nTx, int nTy) {
  BinGroups r;
  r.gh = 1;
  const long long rows_all = (long long)B * nTy;
  int c = 1;
  if (rows_all < kBinRowTargetGroups && nTx >= 2 * kBinMinChunkTiles) {
    c = (int)((kBinRowTargetGroups + rows_all - 1) / rows_all);
    if (c > nTx / kBinMinChunkTiles) c = nTx / kBinMinChunkTiles;
  }
  r.cw = (nTx + c - 1) / c;
  r.ncc = (nTx + r.cw - 1) / r.cw;
  long long nc = ((long long)N + 63) / 64 * 64;
  if (nc > kMaxChunk) nc = kMaxChunk;
  const long long row_max = kBinLdsBytes * 8 / (r.cw + 32) / 64 * 64;
  if (nc > row_max) nc = row_max;
  r.NC = (int)nc;
  r.G = nTy * r.ncc;
  return r;
}

// Two-level binning where the one-level member scan would dominate: many
// Gaussians per frame and a frame cut into many groups, each of which would
// scan all of the frame's boxes.  The row pass holds a bit matrix of every
// tile row against RB Gaussians (RB a multiple of 64 between kBinRowBlockMin
// and kBinRowBlock, smaller when the LDS holds fewer columns).
RowPlan row_plan(int B, int N, int H, int W) {
  RowPlan rp;
  rp.on = false;
  rp.RB = rp.nblk = 0;
  rp.B = B;
  const int nTx = (W + kTileW - 1) / kTileW, nTy = (H + kTileH - 1) / kTileH;
  rp.nTy = nTy;
  if (kBinRows == 0) return rp;
  if (kBinRows < 0) {
    if (N < kBinRowsMinN) return rp;
    if (!member_rule(N, choose_groups(B, N, nTx, nTy, false))) return rp;
  }
  // blocks small enough for about kBinRowBlocks workgroups over the batch
  long long rb = (long long)N * B / kBinRowBlocks / 64 * 64;
  if (rb < kBinRowBlockMin) rb = kBinRowBlockMin;
  if (rb > kBinRowBlock) rb = kBinRowBlock;
  const long long rb_lds = kBinLdsBytes * 8 / nTy / 64 * 64;
  if (rb > rb_lds) rb = rb_lds;
  if (rb < 64) return rp;
  rp.RB = (int)rb;
  rp.nblk = (N + rp.RB - 1) / rp.RB;
  rp.on = true;
  return rp;
}

// The binning variant of a problem, decided from (B, N, H, W) alone.
struct BinPlan {
  RowPlan rp;     // two-level when rp.on
  BinGroups bg;   // the (second-level) groups
  bool members;   // member chunks (always with rp.on)
};

static BinPlan plan_binning(int B, int N, int H, int W) {
  BinPlan p;
  const int nTx = (W + kTileW - 1) / kTileW, nTy = (H + kTileH - 1) / kTileH;
  p.rp = row_plan(B, N, H, W);
  if (p.rp.on) {
    p.bg = row_groups(B, N, nTx, nTy);
    p.members = true;
    return p;
  }
  p.bg = choose_groups(B, N, nTx, nTy, false);
  p.members = kBinMembers > 0 || (kBinMembers < 0 && member_rule(N, p.bg));
  if (p.members) p.bg = choose_groups(B, N, nTx, nTy, true);
  return p;
}

int bin_variant(int B, int N, int H, int W) {
  const BinPlan p = plan_binning(B, N, H, W);
  return (p.members ? 1 : 0) | (p.bg.ncc > 1 ? 2 : 0) | (p.rp.on ? 4 : 0);
}

hipError_t launch_preprocess(const float *params, int B, int N, int H, int W, int C, float radius,
                             void *ws, const Layout &L, bool stamp_valid, hipStream_t st) {
  char *w = (char *)ws;
  long long BN = (long long)B * N;
  const bool ordered = tile_order_on((long long)B * ((W + kTileW - 1) / kTileW) *
                                     ((H + kTileH - 1) / kTileH));
  const long long blocks = std::max((BN + 255) / 256, ordered ? (long long)kZeroBlocks : 1LL);
  PDR_TIMED(PDR_K_PREPROCESS, st,
            hipLaunchKernelGGL(k_preprocess, dim3((unsigned)blocks), dim3(256), 0, st,
                               params, (int)BN, C, make_fastdiv((uint32_t)(5 + C)), H, W, radius,
                               (GRec *)(w + L.recs), (ThinRec *)(w + L.thin),
                               (uint2 *)(w + L.boxes), (WsHeader *)(w + L.hdr), N,
                               stamp_valid ? (unsigned long long)(uintptr_t)params : 0ull,
                               ordered ? (int *)(w + L.ohist) : (int *)nullptr));
  return hipGetLastError();
}

hipError_t launch_binning(const float *params, int B, int N, int H, int W, int C, float radius,
                          void *ws, const Layout &L, int *tile_off, int *list, long long cap,
                          bool stamp_valid, hipStream_t st) {
  char *w = (char *)ws;
  WsHeader *hdr = (WsHeader *)(w + L.hdr);
  GRec *recs = (GRec *)(w + L.recs);
  uint2 *boxes = (uint2 *)(w + L.boxes);
  int *counts = (int *)(w + L.counts);
  int *gtot = (int *)(w + L.gtot);
  long long BN = (long long)B * N;
  int nTx = (W + kTileW - 1) / kTileW, nTy = (H + kTileH - 1) / kTileH;
  const bool ordered = tile_order_on((long long)B * nTx * nTy);
  int *ohist = ordered ? (int *)(w + L.ohist) : nullptr;
  int *order = ordered ? (int *)(w + L.order) : nullptr;
  const hipError_t pe = launch_preprocess(params, B, N, H, W, C, radius, ws, L, stamp_valid, st);
  if (pe != hipSuccess) return pe;
  const BinPlan plan = plan_binning(B, N, H, W);
  const RowPlan &rp = plan.rp;
  if (rp.on) {
    // rows: count, scan, write the per-row lists; then each tile row's
    // tiles from its row's list (member chunks)
    int *rcnt = (int *)(w + L.rcnt), *fstart = (int *)(w + L.fstart), *rlist = (int *)(w + L.rlist);
    const BinGroups &bg = plan.bg;
    if (bg.NC < 64 || bg.NC % 64 != 0) return hipErrorInvalidValue;
    const dim3 g1((unsigned)xcd_grid(rp.nblk, B)), g2((unsigned)xcd_grid(bg.G, B));
    const size_t lds1 = (size_t)nTy * (rp.RB / 32) * 4;
    const size_t lds2 = (size_t)bg.cw * (bg.NC / 32) * 4 + (size_t)bg.NC * 4;
    const bool cols = bg.ncc > 1;
    auto k_rcount = k_rows<false>;
    auto k_rwrite = k_rows<true>;
    auto k_count = cols ? k_bin<false, true, true, true> : k_bin<false, true, false, true>;
    auto k_write = cols ? k_bin<true, true, true, true> : k_bin<true, true, false, true>;
    PDR_TIMED(PDR_K_BIN_COUNT, st, {
      hipLaunchKernelGGL(k_rcount, g1, dim3(kBinThreads), lds1, st, boxes, B, N, nTy, rp.RB,
                         rp.nblk, rcnt, (const int *)fstart, rlist, L.cap);
      hipLaunchKernelGGL(k_rowscan, dim3((unsigned)xcd_grid(nTy, B)), dim3(kWave), 0, st, rcnt,
                         B, nTy, rp.nblk, fstart);
      hipLaunchKernelGGL(k_rowstart, dim3((unsigned)B), dim3(kBinThreads), 0, st, nTy, fstart);
      hipLaunchKernelGGL(k_rwrite, g1, dim3(kBinThreads), lds1, st, boxes, B, N, nTy, rp.RB,
                         rp.nblk, rcnt, (const int *)fstart, rlist, L.cap);
      hipLaunchKernelGGL(k_count, g2, dim3(kBinThreads), lds2, st, boxes, B, N, nTx, nTy, 1,
                         bg.ncc, bg.cw, bg.G, bg.NC, counts, gtot, (int *)nullptr, (int *)nullptr,
                         cap, hdr, ohist, order, (const int *)rlist, (const int *)fstart, L.cap);
    });
    PDR_TIMED(PDR_K_SCAN, st,
              hipLaunchKernelGGL(k_count_scan, dim3(9), dim3(kBinThreads), 0, st, gtot,
                                 (long long)B * bg.G, cap, hdr, ohist,
                                 (unsigned)(B * nTx * nTy)));
    PDR_TIMED(PDR_K_BIN_WRITE, st,
              hipLaunchKernelGGL(k_write, g2, dim3(kBinThreads), lds2, st, boxes, B, N, nTx, nTy,
                                 1, bg.ncc, bg.cw, bg.G, bg.NC, counts, gtot, tile_off, list, cap,
                                 hdr, ohist, order, (const int *)rlist, (const int *)fstart,
                                 L.cap));
    return hipGetLastError();
  }
  const BinGroups &bg = plan.bg;
  const bool members = plan.members;
  if (bg.NC < 64 || bg.NC % 64 != 0) return hipErrorInvalidValue;  // whole 64-column words
  const size_t lds = (size_t)bg.cw * bg.gh * (bg.NC / 32) * 4 + (members ? (size_t)bg.NC * 4 : 0);
  dim3 grid((unsigned)xcd_grid(bg.G, B));
  const bool cols = bg.ncc > 1;
  auto k_count = members ? (cols ? k_bin<false, true, true> : k_bin<false, true, false>)
                         : (cols ? k_bin<false, false, true> : k_bin<false, false, false>);
  auto k_write = members ? (cols ? k_bin<true, true, true> : k_bin<true, true, false>)
                         : (cols ? k_bin<true, false, true> : k_bin<true, false, false>);
  PDR_TIMED(PDR_K_BIN_COUNT, st, {
    hipLaunchKernelGGL(k_count, grid, dim3(kBinThreads), lds, st, boxes, B, N, nTx, nTy, bg.gh,
                       bg.ncc, bg.cw, bg.G, bg.NC, counts, gtot, (int *)nullptr, (int *)nullptr,
                       cap, hdr, ohist, order, (const int *)nullptr, (const int *)nullptr, 0LL);
  });
  PDR_TIMED(PDR_K_SCAN, st,
            hipLaunchKernelGGL(k_count_scan, dim3(9), dim3(kBinThreads), 0, st, gtot,
                               (long long)B * bg.G, cap, hdr, ohist, (unsigned)(B * nTx * nTy)));
  PDR_TIMED(PDR_K_BIN_WRITE, st,
            hipLaunchKernelGGL(k_write, grid, dim3(kBinThreads), lds, st, boxes, B, N, nTx, nTy,
                               bg.gh, bg.ncc, bg.cw, bg.G, bg.NC, counts, gtot, tile_off, list, cap,
                               hdr, ohist, order, (const int *)nullptr, (const int *)nullptr,
                               0LL));
  return hipGetLastError();
}

}  // namespace pdr
