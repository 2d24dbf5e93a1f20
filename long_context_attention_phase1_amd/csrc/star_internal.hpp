// Internal declarations shared by the host runtime (star_host.cpp) and the
// HIP kernels (star_kernels.hip). Not part of the public ABI.
#pragma once

#include <stdint.h>

#include "../../include/star_attn.h"

namespace star {

constexpr int kTile = STAR_KV_TILE;   // rows of a KV-cache tile
constexpr int kWaves = 4;             // waves per workgroup of the MFMA kernels
constexpr int kColsPerWave = 64;      // query columns (row, head pairs) per wave
constexpr int kNarrowCols = 32;       // columns of the single-tile decode kernel
constexpr int kTargetWorkgroups = 256;   // phase-2 planner target, many query rows (one per CU:
                                         // fewer, longer splits write fewer fp32 partials)
constexpr int kNarrowWorkgroups = 256;   // phase-2 planner target, decode (one per CU)
constexpr int kDecodeWaves = 4 * 256;    // balanced plan: ranges per launch (4 waves per CU)
constexpr int kSlice = 32;               // balanced plan: ranges are whole 32-key slices
constexpr int kMinRange = 128;           // balanced plan: shortest range

// Everything derived from a validated descriptor.
struct Dims {
  int32_t B, Hq, Hkv, G, D;
  int64_t L, blk, anc, tail_cap, rows;  // rows: cache rows per (seq, kv head)
  int32_t n_blocks;
  int32_t dtype;
  float scale;      // softmax scale
  float scale_log2; // scale * log2(e)
  // MFMA kernels: heads per workgroup (HW), 64-row sub-tiles per workgroup
  // (RW = 4 / HW), head sub-groups per kv head (HQ = G / HW).
  int32_t HW, RW, HQ;
};

// Phase-2 split plan: every split lies inside one host's share.
//
// Blockwise plan: each context block is cut into per_block splits of
// blk_len rows and the tail into tail_splits of tail_len rows; one workgroup
// per split.
//
// Balanced plan (decode kernel, bf16): the rows [0, kv_len) of every
// (sequence, kv head) are cut into n_wg equal ranges of wg_rows rows (whole
// 32-key slices), one wave each, four waves per workgroup, so that the whole
// grid is resident at once. A range holds at most one host boundary (a block
// start, or the context/tail edge), anywhere in it, on a slice edge or not;
// a range that holds one yields two splits, one on each side. Splits are
// numbered in row order.
struct Plan {
  int32_t narrow;         // 1: single-column-tile decode kernel, 0: wide kernel
  int32_t per_block;      // splits per context block
  int64_t blk_len;        // rows per block split
  int32_t tail_splits;    // splits of the tail [L, kv_len)
  int64_t tail_len;       // rows per tail split
  int32_t n_split;
  int32_t n_groups;       // workgroup groups (sequence, kv head[, head sub-group])
  int32_t n_qtiles;       // query-row tiles (wide kernel)
  int32_t balanced;       // 1: balanced plan
  int32_t n_wg;           // balanced: ranges (waves) per group
  int64_t wg_rows;        // balanced: rows per range
  int64_t bnd_period;     // balanced: block starts i*blk with i % bnd_period == 0 fall on a range edge
};

int validate_desc(const star_attn_desc* d, Dims* out);
int validate_phase2(const Dims& d, int64_t kv_len, int64_t n_query);
Plan make_plan(const Dims& d, int64_t kv_len, int64_t n_query);

#if defined(__HIPCC__)
#define STAR_HD __host__ __device__
#else
#define STAR_HD
#endif

// First host boundary strictly inside (lo, hi), or -1. Host boundaries are
// the block starts i*blk (1 <= i < n_blocks) and the tail start L.
STAR_HD static inline int64_t inner_boundary(int64_t L, int64_t blk, int32_t n_blocks, int64_t lo,
                                             int64_t hi) {
  const int64_t i = lo / blk + 1;
  if (i <= (int64_t)n_blocks - 1 && i * blk < hi) return i * blk;
  if (L > lo && L < hi) return L;
  return -1;
}

// Balanced plan: number of host boundaries below x that do not fall on a
// range edge (each adds one split before x).
STAR_HD static inline int64_t inner_boundaries_below(int64_t L, int64_t blk, int32_t n_blocks,
                                                     int64_t wg_rows, int64_t bnd_period,
                                                     int64_t x) {
  if (x <= 0) return 0;
  int64_t m = (x - 1) / blk;
  if (m > (int64_t)n_blocks - 1) m = (int64_t)n_blocks - 1;
  int64_t c = m - m / bnd_period;
  if (L < x && L % wg_rows != 0) ++c;
  return c;
}

// Split sigma of a plan -> rows [lo, hi) (lo == hi: empty) and host id
// (context block index, or n_blocks for the tail).
STAR_HD static inline void split_rows(int64_t L, int64_t blk, int32_t n_blocks, int32_t per_block,
                                      int64_t blk_len, int64_t tail_len, int64_t kv_len,
                                      int32_t sigma, int64_t* lo, int64_t* hi, int32_t* host) {
  const int64_t nb = (int64_t)n_blocks * per_block;
  if (sigma < nb) {
    const int64_t i = sigma / per_block, j = sigma % per_block;
    const int64_t bend = (i + 1) * blk < L ? (i + 1) * blk : L;
    int64_t a = i * blk + j * blk_len, b = a + blk_len;
    if (b > bend) b = bend;
    if (a > b) a = b;
    *lo = a; *hi = b; *host = (int32_t)i;
  } else {
    const int64_t t = sigma - nb;
    int64_t a = L + t * tail_len, b = a + tail_len;
    if (b > kv_len) b = kv_len;
    if (a > b) a = b;
    *lo = a; *hi = b; *host = n_blocks;
  }
}

static inline void split_range(const Dims& d, const Plan& p, int64_t kv_len, int32_t sigma,
                               int64_t* lo, int64_t* hi, int32_t* host) {
  if (!p.balanced) {
    split_rows(d.L, d.blk, d.n_blocks, p.per_block, p.blk_len, p.tail_len, kv_len, sigma, lo, hi,
               host);
    return;
  }
  // balanced plan: walk the ranges in row order, one or two splits each
  int64_t base = 0;
  for (int64_t j = 0; j < p.n_wg; ++j) {
    const int64_t a = j * p.wg_rows;
    const int64_t b = a + p.wg_rows < kv_len ? a + p.wg_rows : kv_len;
    const int64_t bnd = inner_boundary(d.L, d.blk, d.n_blocks, a, b);
    const int64_t n = bnd >= 0 ? 2 : 1;
    if (sigma < base + n) {
      const bool second = sigma == base + 1;
      *lo = second ? bnd : a;
      *hi = (bnd >= 0 && !second) ? bnd : b;
      *host = *lo < d.L ? (int32_t)(*lo / d.blk) : d.n_blocks;
      return;
    }
    base += n;
  }
  *lo = *hi = kv_len;
  *host = d.n_blocks;
}

// ---- launch geometry and workgroup -> work maps
//
// Shared by the kernels (which call the STAR_HD maps on blockIdx) and by the
// host replay in the tests, which walks every workgroup of a launch through
// the same functions and checks that every work item is done once and every
// address lies inside its buffer.

constexpr int kXcds = 8;       // MI355X: accelerator complex dies, one L2 each;
                               // workgroup i of a launch runs on XCD i % 8
constexpr int kWideWaves = 8;  // waves per wide-kernel workgroup (two per SIMD)

STAR_HD static inline int64_t cdiv_hd(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Wide-kernel launch: NG groups (sequence, kv head, head sub-group) times NRT
// row tiles of BM rows (phase 1: of every block; phase 2: of the query rows)
// times n_blocks blocks (phase 1) or n_split splits (phase 2).
struct WideGeom {
  int32_t phase1;
  int32_t NG, NRT, BM, HQ;
  int32_t n_blocks, n_split;
  int64_t grid;  // workgroups
};

static inline WideGeom phase1_geom(const Dims& d) {
  WideGeom g{};
  g.phase1 = 1;
  g.HQ = d.HQ;
  g.BM = kColsPerWave * d.RW;
  g.NG = d.B * d.Hkv * d.HQ;
  g.NRT = (int32_t)cdiv_hd(d.blk, g.BM);
  g.n_blocks = d.n_blocks;
  g.n_split = 0;
  g.grid = (int64_t)g.NG * d.n_blocks * g.NRT;
  return g;
}

static inline WideGeom wide2_geom(const Dims& d, const Plan& p) {
  WideGeom g{};
  g.phase1 = 0;
  g.HQ = d.HQ;
  g.BM = kColsPerWave * d.RW;
  g.NG = p.n_groups;
  g.NRT = p.n_qtiles;
  g.n_blocks = d.n_blocks;
  g.n_split = p.n_split;
  g.grid = (int64_t)g.NG * g.NRT * p.n_split;
  return g;
}

// Wide kernel: workgroup bid -> (group gidx, work item). bid % NG keeps a
// group on one XCD. With more groups than XCDs (several sequences, or head
// sub-groups) each XCD runs its groups one after another, so its L2 holds
// one group's K/V at a time. In phase 2, where the head sub-groups and query
// tiles of a kv head read the same split, an XCD takes every work item of a
// kv head, with the readers of one split next to each other (so they run at
// the same time).
STAR_HD static inline void wide_map(int64_t bid, bool phase1, int32_t NG, int32_t HQ, int32_t NRT,
                                    int32_t n_split, int32_t n_blocks, int32_t* gidx,
                                    int64_t* work) {
  if (!phase1 && HQ * NRT > 1 && (NG / HQ) % kXcds == 0) {
    const int64_t per_kv = (int64_t)HQ * NRT * n_split;
    const int64_t i = bid / kXcds, r = i % per_kv;
    *gidx = ((int32_t)(bid % kXcds) + kXcds * (int32_t)(i / per_kv)) * HQ + (int32_t)(r % HQ);
    *work = r / HQ;
  } else if (NG > kXcds && NG % kXcds == 0) {
    const int64_t per_group = phase1 ? (int64_t)n_blocks * NRT : (int64_t)NRT * n_split;
    const int64_t i = bid / kXcds;
    *gidx = (int32_t)(bid % kXcds) + kXcds * (int32_t)(i / per_group);
    *work = i % per_group;
  } else {
    *gidx = (int32_t)(bid % NG);
    *work = bid / NG;
  }
}

// fp32 MFMA kernel: one workgroup per 32 columns.
// Phase 1: workgroup -> (sequence s, head h, row group rg); its columns are the
// context rows 32 rg .. 32 rg + 31 of head h.
STAR_HD static inline void f32m_phase1_map(int64_t wid, int64_t L, int32_t Hq, int64_t* s,
                                           int32_t* h, int64_t* rg) {
  const int64_t nrg = cdiv_hd(L, 32);
  *rg = wid % nrg;
  const int64_t t = wid / nrg;
  *h = (int32_t)(t % Hq);
  *s = t / Hq;
}
// Phase 2: workgroup -> (sequence s, kv head kvh, column group cg, split sigma);
// column c of group cg is query row (32 cg + c) / G of head kvh * G + (32 cg + c) % G.
STAR_HD static inline void f32m_phase2_map(int64_t wid, int32_t n_split, int64_t ncg, int32_t Hkv,
                                           int64_t* s, int32_t* kvh, int64_t* cg,
                                           int32_t* sigma) {
  *sigma = (int32_t)(wid % n_split);
  int64_t t = wid / n_split;
  *cg = t % ncg;
  t /= ncg;
  *kvh = (int32_t)(t % Hkv);
  *s = t / Hkv;
}
// Column c (0..31) of an fp32 MFMA workgroup: its row of q, head, whether it is a
// live column, and the keys it sees: [0, hiA) and [loB, hiB) (phase 1: the
// anchor for blocks >= 1, then its block causally; phase 2: split rows
// [lo, hi) up to its own position). Phase 1: rg is the row group and h the
// head; phase 2: cg is the column group and h the kv head.
struct F32mCol {
  int64_t row, hiA, loB, hiB;
  int32_t head;
  bool valid;
};
STAR_HD static inline F32mCol f32m_column(bool phase1, int c, int64_t rg_or_cg, int32_t h,
                                          int64_t L, int64_t blk, int64_t anc, int64_t q_tokens,
                                          int32_t G, int64_t kv_len, int64_t lo, int64_t hi) {
  F32mCol x;
  if (phase1) {
    x.row = rg_or_cg * 32 + c;
    x.head = h;
    x.valid = x.row < L;
    const int64_t i = x.valid ? x.row / blk : 0;
    x.hiA = i > 0 ? anc : 0;
    x.loB = i * blk;
    x.hiB = x.row + 1;
  } else {
    const int64_t cc = rg_or_cg * 32 + c;
    x.row = cc / G;
    x.head = (int32_t)(h * G + cc % G);
    x.valid = x.row < q_tokens;
    const int64_t pos = kv_len - q_tokens + x.row;
    x.hiA = 0;
    x.loB = lo;
    x.hiB = hi < pos + 1 ? hi : pos + 1;
  }
  return x;
}
// The keys an fp32 MFMA workgroup loads: [0, kA) and [kB0, kB1), the union of its
// live columns' ranges; a 32-key slice [k0, k0 + 32) is processed when it
// meets them (f32m_slice).
STAR_HD static inline void f32m_wave_keys(bool phase1, int64_t rg_or_cg, int32_t h, int64_t L,
                                          int64_t blk, int64_t anc, int64_t q_tokens, int32_t G,
                                          int64_t kv_len, int64_t lo, int64_t hi, int64_t* kA,
                                          int64_t* kB0, int64_t* kB1) {
  *kA = 0;
  *kB0 = INT64_MAX;
  *kB1 = 0;
  for (int c = 0; c < 32; ++c) {
    const F32mCol x = f32m_column(phase1, c, rg_or_cg, h, L, blk, anc, q_tokens, G, kv_len, lo, hi);
    if (!x.valid) continue;
    if (x.hiA > *kA) *kA = x.hiA;
    if (x.hiB > x.loB) {
      if (x.loB < *kB0) *kB0 = x.loB;
      if (x.hiB > *kB1) *kB1 = x.hiB;
    }
  }
}
STAR_HD static inline bool f32m_slice(int64_t k0, int64_t kA, int64_t kB0, int64_t kB1) {
  return k0 < kA || (k0 + 32 > kB0 && k0 < kB1);
}
// The same slices in closed form, in order: the nA slices of [0, kA), then
// the block slices from bf up to kB1; slice i starts at f32m_slice_at(i).
struct F32mSlices {
  int64_t nA, bf, n;
};
STAR_HD static inline F32mSlices f32m_slices(int64_t kA, int64_t kB0, int64_t kB1) {
  F32mSlices r;
  r.nA = cdiv_hd(kA, 32);
  const bool any_b = kB1 > kB0;
  const int64_t bl = any_b ? cdiv_hd(kB1, 32) : 0;
  r.bf = any_b ? kB0 / 32 : 0;
  if (r.bf < r.nA) r.bf = r.nA;
  r.n = r.nA + (bl > r.bf ? bl - r.bf : 0);
  return r;
}
STAR_HD static inline int64_t f32m_slice_at(const F32mSlices& sl, int64_t i) {
  return 32 * (i < sl.nA ? i : sl.bf + (i - sl.nA));
}
// Waves per fp32 workgroup: its 32 columns' slices are dealt round robin to
// them (the LDS holds a K, V and P buffer per wave).
STAR_HD constexpr int f32m_waves(int D) { return D <= 64 ? 4 : 2; }
static inline int64_t f32m_ncg(const Dims& d, int64_t n_query) {
  return cdiv_hd(n_query * d.G, 32);
}
static inline int64_t f32m_phase1_grid(const Dims& d) {
  return (int64_t)d.B * d.Hq * cdiv_hd(d.L, 32);
}
static inline int64_t f32m_phase2_grid(const Dims& d, const Plan& p, int64_t n_query) {
  return (int64_t)d.B * d.Hkv * f32m_ncg(d, n_query) * p.n_split;
}

// Phase 2 on the wide kernel: one query tile with at most half its rows live
// (the waves holding the other half only load tiles and meet barriers).
static inline bool wide2_short(const WideGeom& g, int64_t n_query) {
  return g.NRT == 1 && 2 * n_query <= g.BM;
}

// Phase 1: work item -> (block i, row tile rt). Anchored blocks go first, one
// after another, each by descending row tile (the heaviest first), then
// block 0: the workgroups an XCD runs at once are neighbouring row tiles of
// one block and share the anchor's and the block's K/V tiles in its L2.
STAR_HD static inline void phase1_item(int64_t work, int32_t n_blocks, int32_t NRT, int64_t* i,
                                       int64_t* rt) {
  const int64_t n1 = (int64_t)(n_blocks - 1) * NRT;
  if (work < n1) {
    *rt = NRT - 1 - work % NRT;
    *i = 1 + work / NRT;
  } else {
    *rt = NRT - 1 - (work - n1);
    *i = 0;
  }
}

// The 64-key tiles one workgroup reads. Anchor keys [0, hiA): interior tiles
// [0, nAi), plus edge tile nAi when hiA is not a multiple of 64. Block keys
// [loB, hiB), causal: interior tiles [i0, i1), whose 64 keys all lie in
// [loB, hiB) at or before min_pos (the earliest query position of the
// workgroup), so every column sees them unmasked; edge tiles [bf, i0) and
// [i1, bl), masked per key.
struct TileRuns {
  int64_t nAi, bf, bl, i0, i1;
  int32_t a_edge;
};

STAR_HD static inline TileRuns tile_runs(int64_t hiA, int64_t loB, int64_t hiB, int64_t min_pos) {
  TileRuns t{};
  t.nAi = hiA / 64;
  t.a_edge = (hiA % 64) != 0;
  if (hiB > loB) {
    t.bf = loB / 64;
    t.bl = cdiv_hd(hiB, 64);
    int64_t t1 = hiB / 64;
    const int64_t tp = (min_pos + 1) / 64;
    if (tp < t1) t1 = tp;
    const int64_t t0 = cdiv_hd(loB, 64);
    t.i0 = t0 > t.bf ? t0 : t.bf;
    t.i1 = t1 < t.bl ? t1 : t.bl;
    if (t.i1 < t.i0) t.i1 = t.i0;
  }
  return t;
}

// Wide kernel, wave w of a workgroup -> its first query row (relative to the
// workgroup's first row) and the head hw (of the HW heads of the workgroup)
// of its 32*QT columns: WPR = 2/QT waves share one 64-row sub-tile of one head.
// Short query tile (phase 2, QT = 1, at most half the rows live): wave w takes
// rows 32*(w / HW) of head w % HW, so waves 4..7, which share SIMDs with
// waves 0..3, hold the idle rows.
STAR_HD static inline void wide_wave(int w, int QT, int HW, bool short_tile, int* hw,
                                     int64_t* row_off) {
  if (short_tile) {
    *hw = w % HW;
    *row_off = (int64_t)(w / HW) * 32;
    return;
  }
  const int WPR = 2 / QT;
  const int wsub = w % WPR, wh = w / WPR;  // 32*QT-row piece, (head, 64-row sub-tile)
  *hw = wh % HW;
  *row_off = (int64_t)(wh / HW) * 64 + wsub * 32 * QT;
}

// Decode kernel (balanced plan): four waves per workgroup, one range each;
// WPG workgroups per (sequence, kv head) group.
static inline int64_t decode_grid(const Dims& d, const Plan& p, int32_t* wpg) {
  *wpg = (p.n_wg + 3) / 4;
  return (int64_t)d.B * d.Hkv * *wpg;
}

// Workgroup bid, wave w -> group gidx and range r (r >= n_wg: no range, the
// wave exits). The workgroups holding the last ranges (the tail and the
// appended rows) start first.
STAR_HD static inline void decode_map(int64_t bid, int w, int32_t NG, int32_t WPG, int32_t* gidx,
                                      int64_t* r) {
  *gidx = (int32_t)(bid % NG);
  *r = (int64_t)(WPG - 1 - (int32_t)(bid / NG)) * 4 + w;
}

// Range r of the balanced plan: rows [lo, hi), the host boundary bnd inside
// it (or -1), its first split sigma (sigma + 1 starts at bnd), its 32-key
// slices n_sl, and n_in, the leading slices every query column sees whole.
struct DecodeRange {
  int64_t lo, hi, bnd;
  int32_t sigma, n_sl, n_in;
};

STAR_HD static inline DecodeRange decode_range(int64_t r, int64_t wg_rows, int64_t kv_len, int64_t L,
                                               int64_t blk, int32_t n_blocks, int64_t bnd_period,
                                               int64_t pos0) {
  DecodeRange d{};
  d.lo = r * wg_rows;
  d.hi = d.lo + wg_rows < kv_len ? d.lo + wg_rows : kv_len;
  d.bnd = inner_boundary(L, blk, n_blocks, d.lo, d.hi);
  d.sigma = (int32_t)(r + inner_boundaries_below(L, blk, n_blocks, wg_rows, bnd_period, d.lo));
  d.n_sl = (int32_t)((d.hi - d.lo + 31) / 32);
  const int64_t vis = pos0 + 1 < d.hi ? pos0 + 1 : d.hi;
  d.n_in = vis > d.lo ? (int32_t)((vis - d.lo) / 32) : 0;
  return d;
}

// Narrow kernel (blockwise plan): workgroup bid -> group gidx and split
// sigma, splits in reverse order (the short, partly masked tail splits start
// first).
STAR_HD static inline void narrow_map(int64_t bid, int32_t NG, int32_t n_split, int32_t* gidx,
                                      int32_t* sigma) {
  *gidx = (int32_t)(bid % NG);
  *sigma = n_split - 1 - (int32_t)(bid / NG);
}

// A decode step whose append runs inside the partial kernel: bf16 and at
// most 32 query columns (the decode kernels, where the one workgroup that
// holds the new rows is their only reader). Otherwise the append is a
// kv_write launch of its own. (Appending inside the wide kernel of a query
// step, whose splits also have one reader each, measured slower: that
// split's workgroup starts after the first 256 and carries the append on the
// launch's critical path.)
static inline bool fused_append(const Dims& d, const Plan& p) {
  return d.dtype == STAR_BF16 && p.narrow;
}

// ---- grid sizes of every launch, checked before a call enqueues anything
//
// HIP takes a grid as a 32-bit count of work-items: a launch whose
// workgroups would not fit is refused (STAR_ERR_SHAPE) rather than
// truncated. The entry points check every grid of a call before its first
// launch, so a call that fails writes nothing.
static inline bool grid_fits(int64_t wgs, int threads) {
  return wgs >= 1 && wgs <= (int64_t)0xFFFFFFFF / threads;
}

// kv_write: one 256-thread workgroup per (64-row tile touched, sequence, kv head)
static inline int64_t kv_write_grid(const Dims& d, int64_t pos0, int64_t n_tok) {
  return ((pos0 + n_tok - 1) / kTile - pos0 / kTile + 1) * d.B * d.Hkv;
}

// phase 1: bf16 wide kernel (512 threads), or one workgroup per 32 rows of a head (fp32)
static inline bool phase1_fits(const Dims& d) {
  if (d.dtype == STAR_F32) return grid_fits(f32m_phase1_grid(d), 64 * f32m_waves(d.D));
  return grid_fits(phase1_geom(d).grid, 64 * kWideWaves);
}

// phase-2 partials under plan p
static inline bool partial_fits(const Dims& d, const Plan& p, int64_t n_query) {
  if (d.dtype == STAR_F32) return grid_fits(f32m_phase2_grid(d, p, n_query), 64 * f32m_waves(d.D));
  if (p.narrow && p.balanced) {
    int32_t wpg;
    return grid_fits(decode_grid(d, p, &wpg), 256);
  }
  if (p.narrow) return grid_fits((int64_t)d.B * d.Hkv * p.n_split, 256);
  return grid_fits(wide2_geom(d, p).grid, 64 * kWideWaves);
}

// the merge: one workgroup per (sequence, query, head) row
static inline bool merge_fits(const Dims& d, int64_t n_query) {
  return grid_fits((int64_t)d.B * n_query * d.Hq, 256);
}

// ---- the no-allocation decode step's scratch: o_part ([rows][n_split][D]
// fp32) at offset 0, lse_part ([rows][n_split] fp32) at the next 256-byte
// boundary, rows = B * n_query * Hq.
static inline int64_t noalloc_lse_offset(const Dims& d, const Plan& p, int64_t n_query) {
  const int64_t o_bytes = (int64_t)d.B * n_query * d.Hq * p.n_split * d.D * 4;
  return (o_bytes + 255) / 256 * 256;
}
static inline bool noalloc_fits(const Dims& d, const Plan& p, int64_t n_query) {
  const int64_t lse_bytes = (int64_t)d.B * n_query * d.Hq * p.n_split * 4;
  return noalloc_lse_offset(d, p, n_query) + lse_bytes <= (int64_t)STAR_NOALLOC_SCRATCH_BYTES;
}

// Device address of the current GPU's scratch (star_kernels.hip): looked up
// once per device, then reused. STAR_OK, or STAR_ERR_HIP.
int scratch_address(void** ptr);

// Kernel launchers (star_kernels.hip). Each returns STAR_OK or STAR_ERR_HIP.
// table / maxp: a paged cache (kc, vc the page pools; table [B][maxp] page
// ids), or null / 0 for the contiguous cache.
// rope_cos / rope_sin: rotary tables [n_pos][D/2] (K rotated at its cache
// row; phase 1's query at its position id, per rope_mode), or null.
int launch_kv_write(const Dims& d, void* kc, void* vc, int64_t pos0, const void* ks,
                    const void* vs, int64_t n_tok, void* stream, const int32_t* table = nullptr,
                    int32_t maxp = 0, const float* rope_cos = nullptr,
                    const float* rope_sin = nullptr);
int launch_phase1(const Dims& d, const void* kc, const void* vc, const void* q, void* o,
                  void* stream, const float* rope_cos = nullptr, const float* rope_sin = nullptr,
                  int rope_mode = 0);
int launch_phase2_partial(const Dims& d, const Plan& p, const void* kc, const void* vc,
                          int64_t kv_len, const void* q, int64_t n_query, float* o_part,
                          float* lse_part, void* stream, const int32_t* table = nullptr,
                          int32_t maxp = 0);
int launch_decode_step(const Dims& d, const Plan& p, void* kc, void* vc, int64_t kv_len,
                       const void* q, const void* k_new, const void* v_new, int64_t n_query,
                       float* o_part, float* lse_part, void* o, int32_t o_dtype, float* lse_out,
                       void* stream, const int32_t* table = nullptr, int32_t maxp = 0);
int launch_lse_merge(const Dims& d, int64_t n_query, int32_t n_split, const float* o_part,
                     const float* lse_part, void* o, int32_t o_dtype, float* lse_out,
                     void* stream);

}  // namespace star
