// pdr_common.hpp -- shared device/host definitions of the gfx950 splatting
// library: workspace layout, per-Gaussian record, wave64 cross-lane helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdr {

// Tile shape in pixels (binning and raster); compile-time tuning knobs.
#ifndef PDR_TILE_SHIFT_X
#define PDR_TILE_SHIFT_X 4
#endif
#ifndef PDR_TILE_SHIFT_Y
#define PDR_TILE_SHIFT_Y 4
#endif
constexpr int kTileShiftX = PDR_TILE_SHIFT_X, kTileShiftY = PDR_TILE_SHIFT_Y;
constexpr int kTileW = 1 << kTileShiftX, kTileH = 1 << kTileShiftY;
constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kBinThreads = 512; // binning workgroup
constexpr int kMaxHW = 32767;    // pixel boxes are packed as 16-bit coordinates
constexpr int kMaxN = 1 << 22;   // per-frame Gaussian count bound of the scan's int32 partials

// sqrt(log2(e) / 2): whitening rows are scaled by it so that
// exp(-q/2) == exp2(-(z1'^2 + z2'^2)) with z' = kappa * z.
constexpr double kKappa = 0.84932180028801904272150283410289;
constexpr double kKappa2 = 0.72134752044448170367996234050095;  // log2(e) / 2

// The whitening rows in fp64, scaled by kappa: [[c/s1, s/s1], [-s/s2, c/s2]]
// (c, s = cos, sin of theta, also returned).  Preprocessing rounds them to
// fp32 for the per-Gaussian records; the compensated evaluation of thin
// Gaussians recomputes them with the same expressions to recover the
// rounding residues.
__device__ __forceinline__ void whitening_rows(float th, float s1, float s2, double *L, double *sn,
                                               double *cs) {
  sincos((double)th, sn, cs);
  const double i1 = kKappa / (double)s1, i2 = kKappa / (double)s2;
  L[0] = *cs * i1;
  L[1] = *sn * i1;
  L[2] = -*sn * i2;
  L[3] = *cs * i2;
}

// Thin Gaussians.  In single precision z = L (p - mu) carries an absolute
// error of order u |L| |p - mu|, and for a Gaussian of anisotropy R the thin
// axis's |L| |p - mu| reaches R k on its support: for R beyond about 10 the
// thin coordinate's error, which rounding of L makes systematic across the
// pixels, moves the theta and thin-scale gradients by more than 1e-4 of
// their value (measured: none above tolerance up to 10:1, some from 12:1).
// Gaussians with row norms |L_2|^2 > 64 |L_1|^2 (anisotropy above 8:1) are
// evaluated with compensation instead:
//  * the mean is split as mu = mh + r with mh a multiple of 2^-8 and
//    |r| <= 2^-9, so p - (mh - o) is exact in fp32 for any pixel centre p
//    relative to an integer origin o while |p - mh + o| < 2^16, and r is
//    folded into a constant per row, c_i = -L_i r (fp64, rounded);
//  * the rows are ordered so that row 2 is the thin one (swapped: the sums
//    of the two rows trade places);
//  * row 2 is evaluated as a float pair: the fp32 row (hi), its fp64
//    rounding residue (lo), and the exact product residue of l22 dy, so its
//    error is u |z2| + O(u^2 |L| |p - mu|).
// Preprocessing writes these constants for every thin Gaussian into a
// per-Gaussian side record; the rasters take them at staging.
constexpr float kThinRatio2 = 64.f;
// The forward image (and the support count, which follows the forward) meets
// its bound with the plain evaluation far beyond that: its terms are the
// weights themselves, whose relative error stays near u R k, and its
// truncation test keeps that error well inside the tie band up to about
// 100:1.  The rasters' forward takes the compensation above 32:1 only.
constexpr float kThinRatio2Fwd = 1024.f;
constexpr double kThinQuantum = 256.0;
constexpr double kThinMaxMean = 16376.0;   // |mh| bound: |p - mh + o| < 2^16 for o, p < 2^15
constexpr int kThinOk = 1, kThinSwap = 2;
struct __attribute__((aligned(16))) ThinRec {
  float mhx, mhy;     // split mean (multiples of 2^-8)
  float lo21, lo22;   // fp64 residues of the thin row
  float c1, c2;       // -L_i r
  int flags;          // kThinOk | kThinSwap
  int pad;
};
static_assert(sizeof(ThinRec) == 32, "thin record is 32 bytes");
// The per-entry part the rasters keep in LDS.
struct ThinX {
  float lo21, lo22, c1, c2;
};

__device__ __forceinline__ bool is_thin(float l11, float l12, float l21, float l22,
                                        float ratio2 = kThinRatio2) {
  const float n1 = l11 * l11 + l12 * l12, n2 = l21 * l21 + l22 * l22;
  const float lo = fminf(n1, n2), hi = fmaxf(n1, n2);
  return hi > ratio2 * lo && hi < 1e30f;
}

// The thin record of a Gaussian with mean (mx, my), fp64 rows L and their
// fp32 roundings l (record order).
__device__ __forceinline__ ThinRec make_thin_rec(float mx, float my, const double *L64,
                                                 const float *l32) {
  ThinRec t{};
  const double hx = rint((double)mx * kThinQuantum) / kThinQuantum;
  const double hy = rint((double)my * kThinQuantum) / kThinQuantum;
  if (!(fabs(hx) <= kThinMaxMean && fabs(hy) <= kThinMaxMean)) return t;   // flags 0: plain
  double L[4] = {L64[0], L64[1], L64[2], L64[3]};
  float l[4] = {l32[0], l32[1], l32[2], l32[3]};
  const bool sw = l[0] * l[0] + l[1] * l[1] > l[2] * l[2] + l[3] * l[3];
  if (sw) {
    double d = L[0]; L[0] = L[2]; L[2] = d;
    d = L[1]; L[1] = L[3]; L[3] = d;
    float f = l[0]; l[0] = l[2]; l[2] = f;
    f = l[1]; l[1] = l[3]; l[3] = f;
  }
  const double rx = (double)mx - hx, ry = (double)my - hy;  // exact, |r| <= 2^-9
  t.mhx = (float)hx;
  t.mhy = (float)hy;
  t.lo21 = (float)(L[2] - (double)l[2]);
  t.lo22 = (float)(L[3] - (double)l[3]);
  t.c1 = (float)(-(L[0] * rx + L[1] * ry));
  t.c2 = (float)(-(L[2] * rx + L[3] * ry));
  t.flags = kThinOk | (sw ? kThinSwap : 0);
  return t;
}

// z' = L (p - mu) of one pixel from d = p - mu (plain), or for a thin
// Gaussian from d = p - mh (exact) with the compensation constants.
template <bool THIN>
__device__ __forceinline__ void whiten(float l11, float l12, float l21, float l22, const ThinX &tx,
                                       float dx, float dy, float &u1, float &u2) {
  if constexpr (THIN) {
    u1 = fmaf(l11, dx, fmaf(l12, dy, tx.c1));
    const float p = l22 * dy;
    const float e = fmaf(l22, dy, -p);  // l22 dy - p, exactly
    const float s = fmaf(l21, dx, p);   // one rounding, relative to the result
    float t = e + tx.c2;
    t = fmaf(tx.lo22, dy, t);
    t = fmaf(tx.lo21, dx, t);
    u2 = s + t;
  } else {
    u1 = l11 * dx + l12 * dy;
    u2 = l21 * dx + l22 * dy;
  }
}

// Status bits raised on the device into the workspace header.
constexpr int kStatusOverflow = 1;
constexpr int kStatusStale = 2;

struct WsHeader {
  int status;        // kStatus* bits of the last call
  int pad0;
  long long total;   // (tile, Gaussian) pairs of the last binning
  long long cap;     // list capacity used by the last binning
  int stamp[8];      // B, N, H, W, C, radius bits, params pointer lo/hi at binning
  int nonfinite;     // the last tile backward met a non-finite dL/dI value
  int pad1[49];
};
static_assert(sizeof(WsHeader) == 256, "header is one 256-byte block");

// Per-Gaussian raster record (32 bytes, two 16-byte loads): mean, the
// whitening rows scaled by kappa, and the packed pixel bounding box.
struct __attribute__((aligned(16))) GRec {
  float mx, my;
  float l11, l12, l21, l22;
  unsigned int bx;  // x0 | x1 << 16, inclusive; x0 > x1 means empty
  unsigned int by;  // y0 | y1 << 16
};
static_assert(sizeof(GRec) == 32, "record is 32 bytes");

constexpr unsigned int kEmptyBox = 0x0000FFFFu;  // x0 = 65535 > x1 = 0

// Rasters take their tiles longest list first within each XCD's share of
// the grid: a counting sort of the tiles by a key made of the list
// length's octave (floor(log2(len + 1)), longest first, 16 classes), its
// quarter of the octave (longest first), the tile's position window in the
// range (kOrderSub windows), then the length within the quarter.  The
// longest tiles of a range -- the ones that would form the tail -- go
// first wherever they are; tiles of similar length sweep the range in
// frame order, which keeps a frame's records together in L2.
#ifndef PDR_ORDER_QUARTERS
#define PDR_ORDER_QUARTERS 4
#endif
#ifndef PDR_ORDER_SUB
#define PDR_ORDER_SUB 16
#endif
#ifndef PDR_ORDER_WINDOW_MAJOR
#define PDR_ORDER_WINDOW_MAJOR 0
#endif
constexpr int kOrderClasses = 16, kOrderSub = PDR_ORDER_SUB, kOrderFine = 512 / PDR_ORDER_SUB;
constexpr int kOrderQ = PDR_ORDER_QUARTERS;   // length steps of an octave taken before the windows
constexpr int kOrderBuckets = kOrderClasses * kOrderSub * kOrderFine;   // keys per XCD range

// Key of a tile with list length len at offset pos of its XCD range of per
// tiles (0 <= key < kOrderBuckets; a longer list never gets a larger key
// within a window).
__device__ __forceinline__ int order_key(int len, unsigned int pos, unsigned int per) {
  const unsigned int l1 = (unsigned int)len + 1u;               // >= 1
  const int cls = min(kOrderClasses - 1, 31 - __clz((int)l1));  // floor(log2(len + 1))
  const unsigned int lo = (1u << cls) - 1u;                     // len in [lo, 2 lo + 1] below the cap
  const int fine = (int)min((unsigned int)kOrderFine - 1u,
                            (((unsigned int)len - lo) * (unsigned int)kOrderFine) >> cls);
  const int sub = (int)(((unsigned long long)pos * kOrderSub) / per);
  constexpr int kF = kOrderFine / kOrderQ;            // fine steps within a quarter
  const int q = fine / kF, f = fine - q * kF;
  if constexpr (PDR_ORDER_WINDOW_MAJOR) {
    return ((sub * kOrderClasses + (kOrderClasses - 1 - cls)) * kOrderQ + (kOrderQ - 1 - q)) * kF +
           (kF - 1 - f);
  }
  return (((kOrderClasses - 1 - cls) * kOrderQ + (kOrderQ - 1 - q)) * kOrderSub + sub) * kF +
         (kF - 1 - f);
}

// The order costs a launch and a histogram clear (~4 us).  It paid at
// 2560 tiles (160 frames of 64x64: both rasters 6-10% faster, though all
// tiles fit the chip at once, the long ones are spread over the CUs first)
// but not at 16 (one 64x64 frame).
constexpr long long kOrderMinTiles = 1024;
inline bool tile_order_on(long long tiles) { return tiles >= kOrderMinTiles; }

// Workspace carve-up; every region starts on a 256-byte boundary.
struct Layout {
  size_t hdr, recs, thin, boxes, counts, gtot, tile_off, order, ohist, list, total;
  size_t rcnt, fstart, rlist;   // per-row member lists (two-level binning only)
  long long cap;
};

// Two-level binning plan: per-row member lists built from blocks of RB
// Gaussians (nblk blocks per frame), then each tile row's tiles from its
// row's list.  Decided on the host from (B, N, H, W) alone.
struct RowPlan {
  bool on;
  int RB, nblk;
  long long B;
  int nTy;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// q = n / d for 0 <= n < 2^31 by multiply and shift (round-up method of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication"): l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1,
// q = (umulhi(n, m) + n) >> l.
struct FastDiv {
  uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
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

// The binning's per-group totals get one slot per tile (a group holds at
// least one tile).  With a row plan, the row counts, row starts and row
// lists follow (the row pairs never exceed the tile pairs, so the list
// capacity serves both).
inline Layout make_layout(long long BN, long long BT, long long cap, const RowPlan &rp) {
  Layout L;
  size_t o = 0;
  L.hdr = o;       o += align256(sizeof(WsHeader));
  L.recs = o;      o += align256(size_t(BN) * sizeof(GRec));
  L.thin = o;      o += align256(size_t(BN) * sizeof(ThinRec));
  L.boxes = o;     o += align256(size_t(BN) * 8);
  L.counts = o;    o += align256(size_t(BT) * 4);
  L.gtot = o;      o += align256(size_t(BT) * 4);
  L.tile_off = o;  o += align256(size_t(BT + 1) * 4);
  L.order = o;     o += align256(size_t(BT) * 4);
  L.ohist = o;     o += align256(size_t(8) * kOrderBuckets * 4);
  L.list = o;      o += align256(size_t(cap) * 4);
  L.rcnt = L.fstart = L.rlist = 0;
  if (rp.on) {
    L.rcnt = o;    o += align256(size_t(rp.B) * rp.nTy * rp.nblk * 4);
    L.fstart = o;  o += align256(size_t(rp.B) * (rp.nTy + 1) * 4);
    L.rlist = o;   o += align256(size_t(cap) * 4);
  }
  L.total = o;
  L.cap = cap;
  return L;
}

// ----------------------------------------------------------------------------
// wave64 cross-lane helpers (DPP / ds_swizzle / ds_bpermute)

// DPP control words (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowRor8 = 0x128;  // within a 16-lane row: lane i <- lane i ^ 8
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Inclusive prefix sum of an int over the 64 lanes of a wave: row_shr steps
// inside each 16-lane row, then row_bcast:15 / row_bcast:31 carry the row
// totals into the rows above.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);
  return v;
}

__device__ __forceinline__ int wave_read(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

// Value of the partner lane (lane ^ MASK), MASK in {1, 2, 4, 8, 16}.
template <int MASK>
__device__ __forceinline__ float xor_partner(float v) {
  int x = __float_as_int(v);
  if constexpr (MASK == 1) {
    x = __builtin_amdgcn_update_dpp(0, x, kDppQuadXor1, 0xF, 0xF, false);
  } else if constexpr (MASK == 2) {
    x = __builtin_amdgcn_update_dpp(0, x, kDppQuadXor2, 0xF, 0xF, false);
  } else if constexpr (MASK == 8) {
    x = __builtin_amdgcn_update_dpp(0, x, kDppRowRor8, 0xF, 0xF, false);
  } else {
    static_assert(MASK == 4 || MASK == 16, "xor_partner mask");
    // ds_swizzle bitmask mode: and 0x1f, or 0, xor MASK (within 32 lanes)
    x = __builtin_amdgcn_ds_swizzle(x, 0x1F | (MASK << 10));
  }
  return __int_as_float(x);
}

// DPP row shift: lane i reads lane i + D of its 16-lane row (lanes whose
// source lies outside the row read 0, bound_ctrl).
template <int D>
__device__ __forceinline__ float dpp_row_shl(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + D, 0xF, 0xF, true));
}

// Sum with the partner lane (lane ^ MASK, MASK in {1, 2, 4, 8, 16}): an
// all-reduce step.
template <int MASK>
__device__ __forceinline__ float xor_sum(float v) {
  return v + xor_partner<MASK>(v);
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

// One exchange step of the transposed butterfly for MASK in {4, 8}, without
// selects: the lanes without the MASK bit are whole DPP banks (4-lane groups
// of a row), so a bank-masked DPP add writes them (own lower-half value plus
// the partner's) and a second one writes the other banks from the upper
// half.  The two instructions write every lane of r once.  Inline asm
// because the compiler forms no DPP add with a partial bank mask.  The
// hazard recognizer does not look into asm, so each block waits two states
// (s_nop 1) before its DPP reads, and the MASK 8 blocks, whose results feed
// the compiler's own DPP steps, also after their write.
template <int MASK>
__device__ __forceinline__ float banked_pair_sum(float lo, float hi) {
  static_assert(MASK == 4 || MASK == 8, "bank-separable lane bits are 2 and 3");
  float r;
  if constexpr (MASK == 4) {
    asm("s_nop 1\n\t"
        "v_add_f32_dpp %0, %1, %1 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
        "v_add_f32_dpp %0, %2, %2 row_shr:4 row_mask:0xf bank_mask:0xa"
        : "=&v"(r)
        : "v"(lo), "v"(hi));
  } else {
    asm("s_nop 1\n\t"
        "v_add_f32_dpp %0, %1, %1 row_shl:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %0, %2, %2 row_shr:8 row_mask:0xf bank_mask:0xc\n\t"
        "s_nop 1"
        : "=&v"(r)
        : "v"(lo), "v"(hi));
  }
  return r;
}

template <int HALF, int MASK>
__device__ __forceinline__ void bstep(float *v) {
#pragma unroll
  for (int i = 0; i < HALF; ++i) v[i] = banked_pair_sum<MASK>(v[i], v[i + HALF]);
}

// Reduce KP per-lane values over the wave.  Transposed steps over the lane
// bits 2, 3 (bank-masked DPP), then 0, 1 (quad_perm DPP with selects) and,
// for KP = 32, 4 (ds_swizzle); the remaining bits are all-reduce steps.
// Afterwards every lane holds the wave total of value value_index<KP>(lane);
// the lanes with reduce_issuer<KP>(lane) hold each value once.
template <int KP>
__device__ __forceinline__ float wave_reduce_transposed(float *v, int lane) {
  static_assert(KP == 8 || KP == 16 || KP == 32, "KP");
  bstep<KP / 2, 4>(v);
  bstep<KP / 4, 8>(v);
  tstep<KP / 8, 1>(v, lane & 1);
  if constexpr (KP >= 16) tstep<KP / 16, 2>(v, lane & 2);
  if constexpr (KP >= 32) tstep<1, 16>(v, lane & 16);
  float r = v[0];
  if constexpr (KP < 16) r = xor_sum<2>(r);
  // the last exchanges through the LDS crossbar (no VALU but the add;
  // measured faster than the permlane swaps): ds_swizzle for lane ^ 16,
  // ds_bpermute for lane ^ 32
  if constexpr (KP < 32) r += xor_partner<16>(r);
  return r + __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(r)));
}

template <int KP>
__device__ __forceinline__ int value_index(int lane) {
  int idx = ((lane & 4) ? KP / 2 : 0) + ((lane & 8) ? KP / 4 : 0) + ((lane & 1) ? KP / 8 : 0);
  if constexpr (KP >= 16) idx += (lane & 2) ? KP / 16 : 0;
  if constexpr (KP >= 32) idx += (lane & 16) ? 1 : 0;
  return idx;
}

// The KP lanes (one per value) whose all-reduce lane bits are zero.
template <int KP>
__device__ __forceinline__ bool reduce_issuer(int lane) {
  constexpr int kAll = KP == 8 ? (2 | 16 | 32) : (KP == 16 ? (16 | 32) : 32);
  return (lane & kAll) == 0;
}

// Blocks of a frame-major grid of (frame, item) pairs.  Workgroups are
// dealt to the 8 XCDs round robin (block i runs on XCD i mod 8), so XCD x
// is given the x-th eighth of the frame-major pair order: a frame's items
// share one L2 (or two, at a range boundary) when frames outnumber XCDs,
// and a frame is spread over several XCDs when they do not.  The grid has
// 8 * ceil(frames * items / 8) blocks; the excess returns false.
__device__ __forceinline__ bool xcd_frame_item(int bid, int items, int frames, int *frame, int *item) {
  const unsigned int total = (unsigned int)items * (unsigned int)frames;
  const unsigned int per = (total + 7u) >> 3;
  const unsigned int lin = (unsigned int)(bid & 7) * per + ((unsigned int)bid >> 3);
  if (lin >= total) return false;
  *frame = (int)(lin / (unsigned int)items);
  *item = (int)(lin - (unsigned int)*frame * (unsigned int)items);
  return true;
}

// The slot of tile lin (of total) in the order histogram: its XCD range
// (xcd_frame_item deals blocks [x per, (x + 1) per) to XCD x) and its key.
__device__ __forceinline__ int order_slot(unsigned int lin, unsigned int total, int len) {
  const unsigned int per = (total + 7u) >> 3;
  const unsigned int r = lin / per;
  return (int)r * kOrderBuckets + order_key(len, lin - r * per, per);
}

// The raster's tile for block bid: the same XCD range as xcd_frame_item, the
// tile taken from the binning's longest-first order of that range.  False
// for the grid's excess blocks (and, defensively, an order entry out of
// range).
__device__ __forceinline__ bool ordered_tile(int bid, int nT, int frames, const int *order,
                                             int *frame, int *tile) {
  const unsigned int total = (unsigned int)nT * (unsigned int)frames;
  const unsigned int per = (total + 7u) >> 3;
  const unsigned int lin = (unsigned int)(bid & 7) * per + ((unsigned int)bid >> 3);
  if (lin >= total) return false;
  const unsigned int tl = (unsigned int)order[lin];
  if (tl >= total) return false;
  *frame = (int)(tl / (unsigned int)nT);
  *tile = (int)(tl - (unsigned int)*frame * (unsigned int)nT);
  return true;
}

// A grid whose items are each split S ways: block bid takes part
// (bid >> 3) % S of the item that block (bid & 7) + 8 ((bid >> 3) / S) of
// the unsplit grid would take, so an item's parts run consecutively on one
// XCD.  Returns that unsplit block index.
__device__ __forceinline__ int split_block(int bid, int S, int *part) {
  const int k = bid >> 3;
  *part = k % S;
  return (bid & 7) | ((k / S) << 3);
}

// Workgroups per tile in the backward raster: one where the tiles fill the
// chip several times over (at 8192 tiles and more, i.e. 8 per SIMD); for
// batches of fewer tiles each tile's list is shared by 2, 4 or 8
// workgroups, so that enough waves are resident to hide the raster's
// latencies.  Measured on MI355X, backward raster: 160 frames of 64x64
// (2560 tiles) 85 -> 48 us with 4, one 64x64 frame 28 -> 9 us with 8;
// from 24576 tiles up one workgroup per tile is as fast or faster.
#ifndef PDR_BWD_SPLITS
#define PDR_BWD_SPLITS 0   // 0: by the number of tiles
#endif
inline int backward_splits(long long tiles) {
  if (PDR_BWD_SPLITS > 0) return PDR_BWD_SPLITS;
  return tiles >= 8192 ? 1 : (tiles >= 4096 ? 2 : (tiles >= 2048 ? 4 : 8));
}

// Waves per tile in the forward raster (the list shared as in the
// backward, the shares' sums added in LDS): the same rule, at most 4.
#ifndef PDR_FWD_SPLITS
#define PDR_FWD_SPLITS 0   // 0: by the number of tiles
#endif
inline int forward_splits(long long tiles) {
  if (PDR_FWD_SPLITS > 0) return PDR_FWD_SPLITS;
  return tiles >= 8192 ? 1 : (tiles >= 4096 ? 2 : 4);
}

inline long long xcd_grid(int items, int frames) {
  return 8LL * (((long long)items * frames + 7) / 8);
}

}  // namespace pdr
